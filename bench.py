#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X.

One step = one whole hot path over the two workloads it serves: msa_prefill
on the 1M-token prefill (batch 1, 1048576 tokens, 64 query / 8 KV heads, head
dim 128, blocks of 128, top_k 16: pooling, index top-k, query->block
inversion, KV-outer attention over every kept block, partial merge, in four
query chunks) followed by one msa_decode of 16 sequences over
262144-token caches (same heads).  Inputs are seeded synthetic tensors
already resident in HBM.  Prints one JSON line; its headline `value` is the
1M prefill's tokens/s.

Beside the step (unless --core-only): the other prefill workloads (2K, 32K,
structured 128K), decode back to back and the generation step, the 32K
prefill in chunks and its training forward/backward, the 1M backward, a
short dense prefill; and (unless --no-cpu-baseline) the CPU oracle timed on
every workload's rows -- all rows of the 2K and 32K prefills and of the
decode, 4096 seeded rows of the 128K and 1M prefills -- with the parity of
those rows against the GPU's.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline] [--core-only]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
D_HEAD = 128
HEADLINE = "prefill_1m"
DECODE = "decode_b16_256k"
CPU_SAMPLE_ROWS = 4096      # oracle rows timed for the 128K and 1M prefills
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_prefill_1m_traffic.json")


def _say(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _prefill_counts(w):
    """Algorithmic work of one prefill: attended keys summed over queries
    (per query head), the part of them in blocks before each query's own
    (the attention kernel's share; the own block's keys go to the merge
    kernel), and the (query row, earlier kept block) pairs."""
    import numpy as np
    t = np.arange(w.seq_len, dtype=np.int64)
    own = t // w.block_size
    kept = np.minimum(w.top_k - 1, own)   # kept blocks before the own one
    earlier_keys = kept * w.block_size
    keys = earlier_keys + (t % w.block_size) + 1
    per_head_keys = int(keys.sum()) * w.batch
    per_head_earlier = int(earlier_keys.sum()) * w.batch
    pairs = int(kept.sum()) * w.batch * w.n_q_heads
    return per_head_keys, per_head_earlier, pairs


def _flop_alg(w):
    return 4.0 * w.head_dim * w.n_q_heads * _prefill_counts(w)[0]


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
    """Hash of the main-branch kernel source; counter records are valid only
    for the source they were taken on."""
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "block_sparse_attention_33_amd", "csrc", "main_branch.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _measured_traffic():
    """HBM bytes per launch of the 1M prefill's attention kernel from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE record (scaled by the copy
    kernel calibration), if it was taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def _median_ms(fn, reps, warm=1):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = _events(reps)
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2]


def _workspace(msa, op, w, dev, cap_bytes=None):
    import torch
    dims = msa.make_dims(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
    lo, hi = msa.msa_workspace_bytes(op, dims)
    size = hi if cap_bytes is None else max(lo, min(hi, cap_bytes))
    return torch.empty(max(size, 256), dtype=torch.uint8, device=dev)


# ------------------------------------------------------------------ counters

def pmc_run():
    """Workload for counter runs under rocprofv3 --pmc: two 1M prefills, two
    decodes of the decode workload, then a 1 GiB device copy whose bytes are
    known (the calibration of the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch
    import block_sparse_attention_33_amd as msa
    from synth import decode_inputs, get_workload, prefill_inputs
    dev = torch.device("cuda:0")
    w = get_workload(HEADLINE)
    inp = prefill_inputs(w, seed=0, device=dev)
    ws = _workspace(msa, msa.MSA_OP_PREFILL, w, dev)
    out = torch.empty_like(inp["q"])
    for _ in range(2):
        msa.msa_prefill(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], w.block_size, w.top_k, out=out,
                        workspace=ws)
    torch.cuda.synchronize()
    del inp, ws, out
    torch.cuda.empty_cache()
    wd = get_workload(DECODE)
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
                m = re.search(r"msa::\(anonymous namespace\)::(\w+(?:<[\w, ]+>)?)", name)
                key = m.group(1) if m else ("copy" if "copyBuffer" in name else None)
                if key:
                    got.setdefault(key, []).append(float(row["Counter_Value"]))
        return got

    fk, wk = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = 2**30 / 1024.0
    fscale, wscale = copy_kib / fk["copy"][-1], copy_kib / wk["copy"][-1]
    rec = {
        "kernel": "attend_kernel<128, true>",
        "workload": "prefill_1m (batch 1, seq 1048576, 64q/8kv heads, head_dim 128, block 128, top_k 16; four "
                    "query chunks of 262144); decode_b16_256k (16 x 262144-token caches, same heads)",
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
    rec["bytes_per_launch"] = rec["attend_kernel<128, true>"]["bytes"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"written": TRAFFIC_FILE, "attend_bytes_per_launch": rec["bytes_per_launch"]}))


def counter_table(stats_csv, pmc_csvs):
    """Markdown table of per-dispatch SQ counters of the MSA kernels from
    rocprofv3 --pmc CSV files (one counter pass each) and the average kernel
    durations of a --kernel-trace --stats run of the same command, with the
    ratios they give.  MI355X: 1024 SIMDs (256 CUs x 4) at 2.4 GHz."""
    import csv
    import re

    def key_of(name):
        m = re.search(r"msa::\(anonymous namespace\)::(\w+(?:<[\w, ]+>)?)", name)
        return m.group(1) if m else None

    dur = {}
    with open(stats_csv, newline="") as f:
        for row in csv.DictReader(f):
            k = key_of(row["Name"])
            if k:
                dur[k] = float(row["AverageNs"]) * 1e-9
    cnt = {}
    for path in pmc_csvs:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                k = key_of(row["Kernel_Name"])
                if k:
                    cnt.setdefault(k, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    simd_cycles = 1024 * 2.4e9
    cols = ["kernel", "avg us", "waves", "VALU / wave", "MFMA / wave", "LDS / wave", "MFMA busy per SIMD",
            "wave cycles waiting on a counter", "waiting for issue", "issuing", "LDS cycles in bank conflicts"]
    print("| " + " | ".join(cols) + " |")
    print("|" + "---|" * len(cols))
    for k in sorted(cnt, key=lambda x: -dur.get(x, 0.0)):
        c = {n: sum(v) / len(v) for n, v in cnt[k].items()}
        g = lambda n: c.get(n)  # noqa: E731

        def ratio(a, b, pct=True):
            if a is None or b is None or b == 0:
                return ""
            return f"{100.0 * a / b:.1f} %" if pct else f"{a / b:.0f}"

        d = dur.get(k)
        mfma_busy = ratio(g("SQ_VALU_MFMA_BUSY_CYCLES"), d * simd_cycles if d else None)
        cells = [k, f"{d * 1e6:.1f}" if d else "", f"{g('SQ_WAVES'):.0f}" if g("SQ_WAVES") else "",
                 ratio(g("SQ_INSTS_VALU"), g("SQ_WAVES"), False), ratio(g("SQ_INSTS_MFMA"), g("SQ_WAVES"), False),
                 ratio(g("SQ_INSTS_LDS"), g("SQ_WAVES"), False), mfma_busy,
                 ratio(g("SQ_WAIT_ANY"), g("SQ_WAVE_CYCLES")), ratio(g("SQ_WAIT_INST_ANY"), g("SQ_WAVE_CYCLES")),
                 ratio(g("SQ_ACTIVE_INST_ANY"), g("SQ_WAVE_CYCLES")),
                 ratio(g("SQ_LDS_BANK_CONFLICT"), g("SQ_LDS_IDX_ACTIVE"))]
        print("| " + " | ".join(cells) + " |")


# ------------------------------------------------------------------ CPU oracle baseline

def _host_info():
    try:
        aff = sorted(os.sched_getaffinity(0))
    except AttributeError:
        aff = None
    return {"cpu_count": os.cpu_count(), "affinity_cpus": len(aff) if aff is not None else None}


def cpu_baseline_prefill(name, inp, out, sel, rows):
    """The oracle (over worker processes, one thread each) on `rows` of a
    prefill workload whose GPU output and selection are given: its rows/s,
    and the parity of those rows."""
    import numpy as np
    import torch
    from oracle import pool
    from synth import get_workload
    w = get_workload(name)
    rt = torch.as_tensor(rows, device=inp["q"].device)
    bits = lambda t: t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    summ, osel, oout, st = pool.prefill_rows(bits(inp["q"][:, rt]), bits(inp["k"]), bits(inp["v"]),
                                             inp["q_idx"].cpu().numpy(), inp["k_idx"].cpu().numpy(), rows,
                                             w.block_size, w.top_k)
    gsel = sel[:, :, rt].cpu().numpy()
    g = out[:, rt].float().cpu().numpy().astype(np.float64)
    d = np.abs(g - oout)
    rel = d.mean(axis=-1) / np.maximum(np.abs(oout).mean(axis=-1), 1e-30)
    return {
        "value": round(len(rows) / st["seconds"], 2), "unit": "tokens/s", "cores": st["workers"], "kind": "oracle",
        "sample": (f"{len(rows)} {'seeded ' if len(rows) < w.seq_len else ''}query positions of {name} "
                   f"(all {w.n_kv_heads} groups, {w.n_q_heads} heads): pooling of all blocks, selection and "
                   f"attention, {st['seconds']:.1f} s over {st['workers']} one-thread worker processes "
                   f"(input files and process start included)"),
        "rows": len(rows), "seconds": st["seconds"], **_host_info(),
        "parity": {"selection_bit_exact": bool(np.array_equal(gsel, osel)), "max_abs": float(d.max()),
                   "mean_abs": float(d.mean()), "max_row_mean_rel": float(rel.max())},
    }


def cpu_baseline_decode(din, block_keys, out, sel, w):
    """The oracle's decode of every (sequence, group) unit, in this process
    (one thread), and the parity of the GPU's decode."""
    import numpy as np
    import torch
    from oracle import msa_oracle as O

    class Bits:  # bf16 cache on the host, gathered rows widened to float32 exactly
        def __init__(self, t):
            self.b = t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
            self.shape = self.b.shape

        def __getitem__(self, idx):
            return (np.asarray(self.b[idx]).astype(np.uint32) << 16).view(np.float32)

    kc, vc = Bits(din["k_cache"]), Bits(din["v_cache"])
    qf = din["q"].float().cpu().numpy()
    qi = din["q_idx"].cpu().numpy()
    summ = block_keys.cpu().numpy()
    t0 = time.perf_counter()
    osel, oout = O.decode(qf, qi, kc, vc, summ, w.block_size, w.top_k)
    dt = time.perf_counter() - t0
    ref = O.round_to_bf16(oout)
    d = np.abs(out.float().cpu().numpy().astype(np.float64) - ref)
    return {
        "value": round(w.batch / dt, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": (f"all {w.batch} sequences x {w.n_kv_heads} groups of {DECODE}: selection over the given "
                   f"summaries and attention, {dt:.2f} s, one thread"),
        "rows": w.batch, "seconds": round(dt, 3), **_host_info(),
        "parity": {"selection_bit_exact": bool(np.array_equal(sel.cpu().numpy(), osel)), "max_abs": float(d.max()),
                   "mean_abs": float(d.mean())},
    }


# ------------------------------------------------------------------ training-only run (profilers)

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
    pws = _workspace(msa, msa.MSA_OP_PREFILL, w, dev)
    bws = _workspace(msa, msa.MSA_OP_BACKWARD, w, dev)

    def fwd():
        return msa.msa_prefill_lse(pin["q"], pin["k"], pin["v"], pin["q_idx"], pin["k_idx"], w.block_size, w.top_k,
                                   workspace=pws)

    out, sel, lse = fwd()

    def bwd():
        return msa.msa_prefill_backward(pin["q"], pin["k"], pin["v"], out, dout, lse, sel, w.block_size,
                                        workspace=bws)

    res = {name: _median_ms(fn, steps, warmup) for name, fn in (("forward_lse", fwd), ("backward", bwd))}
    flop = 2.5 * _flop_alg(w)
    print(json.dumps({"workload": "prefill_32k training", "forward_lse_ms": round(res["forward_lse"], 4),
                      "backward_ms": round(res["backward"], 4),
                      "backward_tflops_alg": round(flop / (res["backward"] * 1e-3) / 1e12, 2)}), flush=True)


# ------------------------------------------------------------------ extras beside the step

def other_prefills(msa, dev, cpu):
    """The 2K, 32K and structured 128K prefills: median time of a few calls,
    and (with cpu) the oracle on their rows with parity."""
    import torch
    from synth import get_workload, prefill_inputs, sample_rows
    res, base = {}, {}
    for name, reps in (("tiny_2k", 10), ("prefill_32k", 10), ("structured_128k", 5)):
        w = get_workload(name)
        inp = prefill_inputs(w, seed=0, device=dev)
        ws = _workspace(msa, msa.MSA_OP_PREFILL, w, dev)
        out = torch.empty_like(inp["q"])
        sel = torch.empty((w.batch, w.n_kv_heads, w.seq_len, w.top_k), dtype=torch.int32, device=dev)

        def fn():
            msa.msa_prefill(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], w.block_size, w.top_k, out=out,
                            sel=sel, workspace=ws)

        ms = _median_ms(fn, reps)
        flop = _flop_alg(w)
        res[name] = {"seq_len": w.seq_len, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                     "block_size": w.block_size, "top_k": w.top_k, "calls": reps, "ms": round(ms, 4),
                     "tokens_per_s": round(w.batch * w.seq_len / (ms * 1e-3), 1),
                     "tflops_alg": round(flop / (ms * 1e-3) / 1e12, 2),
                     "frac_bf16_peak": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        _say(f"{name}: {ms:.3f} ms")
        if cpu:
            rows = sample_rows(w.seq_len, w.seq_len if w.seq_len <= 32768 else CPU_SAMPLE_ROWS, 12345)
            base[name] = cpu_baseline_prefill(name, inp, out, sel, rows)
            _say(f"{name}: oracle {base[name]['value']} tokens/s, parity {base[name]['parity']}")
        del inp, ws, out, sel
        torch.cuda.empty_cache()
    return res, base


def decode_extras(msa, din, block_keys, wd, dws, dout, steps):
    """Decode back to back (the kept blocks may still sit in the memory-side
    cache) and the generation step (append + decode)."""
    import torch
    L = wd.seq_len
    gen_keys, gen_sums = msa.msa_decode_init(din["k_idx_cache"], L - 1, wd.block_size)
    k_new = din["k_cache"][:, :, L - 1].contiguous()
    v_new = din["v_cache"][:, :, L - 1].contiguous()
    k_idx_new = din["k_idx_cache"][:, :, L - 1].contiguous()

    def decode():
        msa.msa_decode(din["q"], din["q_idx"], din["k_cache"], din["v_cache"], block_keys, wd.block_size, wd.top_k,
                       out=dout, workspace=dws)

    def gen_step():
        msa.msa_decode_step(din["q"], din["q_idx"], k_new, v_new, k_idx_new, din["k_cache"], din["v_cache"],
                            gen_sums, gen_keys, L, wd.block_size, wd.top_k, out=dout, workspace=dws)

    b2b = _median_ms(decode, steps, 3) * 1e3
    gen = _median_ms(gen_step, steps, 3) * 1e3
    dbytes = _decode_bytes(wd)
    # the decode captured once in a HIP graph, as a serving loop would run
    # it, and `n` replays enqueued back to back between two events (the GPU
    # never waits for the host); the same for `n` eager calls
    n = max(steps, 20)
    graph, graph_error = None, None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            decode()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode()
        graph.replay()
        torch.cuda.synchronize()
    except RuntimeError as e:  # the record keeps the other numbers
        graph_error = str(e)[:200]
        graph = None

    def queued_us(fn):
        a, b = _events(1)[0]
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    graph_us = queued_us(graph.replay) if graph is not None else None
    queued = queued_us(decode)
    return {"decode_back_to_back_us": round(b2b, 2), "decode_back_to_back_frac_hbm_peak":
            round(dbytes / (b2b * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "decode_graph_replay_us": round(graph_us, 2) if graph_us else None,
            "decode_graph_replay_frac_hbm_peak":
                round(dbytes / (graph_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4) if graph_us else graph_error,
            "decode_queued_us": round(queued, 2),
            "decode_graph_what": f"the decode captured in a HIP graph, {n} replays enqueued back to back between "
                                 "two events (decode_queued_us: the same for eager calls); the kept blocks may "
                                 "still sit in the memory-side cache",
            "generation_step_us": round(gen, 2),
            "generation_step_what": "append one token per sequence (K/V rows, running index-key sum, block "
                                    "summary) + decode, back to back",
            "generation_step_frac_hbm_peak": round(dbytes / (gen * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


def training_extras(msa, dev):
    """The 32K prefill's training forward and backward, and the 1M backward in
    query passes."""
    import torch
    from synth import get_workload, grad_output, prefill_inputs
    res = {}
    w = get_workload("prefill_32k")
    pin = prefill_inputs(w, seed=0, device=dev)
    pws = _workspace(msa, msa.MSA_OP_PREFILL, w, dev)
    bws = _workspace(msa, msa.MSA_OP_BACKWARD, w, dev)
    out, sel, lse = msa.msa_prefill_lse(pin["q"], pin["k"], pin["v"], pin["q_idx"], pin["k_idx"], w.block_size,
                                        w.top_k, workspace=pws)
    dout = grad_output(w, seed=0, device=dev)
    fwd_ms = _median_ms(lambda: msa.msa_prefill_lse(pin["q"], pin["k"], pin["v"], pin["q_idx"], pin["k_idx"],
                                                    w.block_size, w.top_k, workspace=pws), 5)
    msa.profile_read()
    msa.profile_enable(True)
    bwd_ms = _median_ms(lambda: msa.msa_prefill_backward(pin["q"], pin["k"], pin["v"], out, dout, lse, sel,
                                                         w.block_size, workspace=bws), 5)
    msa.profile_enable(False)
    bkt = msa.profile_read()
    flop = 2.5 * _flop_alg(w)
    res["prefill_32k"] = {
        "forward_lse_ms": round(fwd_ms, 4), "backward_ms": round(bwd_ms, 4),
        "backward_tflops_alg": round(flop / (bwd_ms * 1e-3) / 1e12, 2),
        "backward_frac_bf16_peak": round(flop / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "backward_flop_alg": flop,
        "kernels": {k: {"launches": n, "avg_ms": round(ms / max(1, n), 4)} for k, (n, ms) in sorted(bkt.items())}}
    del pin, pws, bws, out, sel, lse, dout
    torch.cuda.empty_cache()
    # 1M backward: the full workspace (about 276 GB) does not fit beside the
    # tensors, so it runs in query passes in 80 % of the free memory
    w = get_workload(HEADLINE)
    cin = prefill_inputs(w, seed=0, device=dev)
    tout, tsel, tlse = msa.msa_prefill_lse(cin["q"], cin["k"], cin["v"], cin["q_idx"], cin["k_idx"], w.block_size,
                                           w.top_k)
    tdout = grad_output(w, seed=0, device=dev)
    torch.cuda.empty_cache()
    dims = msa.make_dims(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
    tlo, thi = msa.msa_workspace_bytes(msa.MSA_OP_BACKWARD, dims)
    tws = torch.empty(max(tlo, min(thi, int(torch.cuda.mem_get_info(dev)[0] * 0.8) - (20 << 30))),
                      dtype=torch.uint8, device=dev)
    msa.profile_read()
    msa.profile_enable(True)
    bms = _median_ms(lambda: msa.msa_prefill_backward(cin["q"], cin["k"], cin["v"], tout, tdout, tlse, tsel,
                                                      w.block_size, workspace=tws), 2)
    msa.profile_enable(False)
    bk1 = msa.profile_read()
    flop = 2.5 * _flop_alg(w)
    rows = msa.msa_backward_pass_rows(dims, tws.numel())
    res[HEADLINE] = {"workspace_gib": round(tws.numel() / 2**30, 1), "passes": -(-w.seq_len // rows),
                     "backward_ms": round(bms, 2), "backward_tflops_alg": round(flop / (bms * 1e-3) / 1e12, 2),
                     "backward_frac_bf16_peak": round(flop / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "bwd_kv_ms_per_call": round(bk1["bwd_kv"][1] / 3, 2) if "bwd_kv" in bk1 else None}
    _say(f"1M backward: {bms:.1f} ms")
    del cin, tout, tsel, tlse, tdout, tws
    torch.cuda.empty_cache()
    return res


def chunked_and_dense(msa, dev):
    """The 32K prefill as four chunks of 8192 queries against the cache, and a
    4096-token prefill with top_k = every block (dense kernel) beside the
    sparse path on the same data."""
    import torch
    from synth import get_workload, prefill_inputs
    res = {}
    w = get_workload("prefill_32k")
    pin = prefill_inputs(w, seed=0, device=dev)
    bounds = [0, 8192, 16384, 24576, w.seq_len]
    cq = [pin["q"][:, a:b].contiguous() for a, b in zip(bounds[:-1], bounds[1:])]
    cqi = [pin["q_idx"][:, :, a:b].contiguous() for a, b in zip(bounds[:-1], bounds[1:])]
    couts = [torch.empty_like(x) for x in cq]
    ckeys = torch.empty((1, w.n_kv_heads, w.seq_len // w.block_size, 64), dtype=torch.int8, device=dev)
    dims = msa.make_dims(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
    cws = torch.empty(msa.msa_prefill_chunk_workspace_bytes(dims, 8192)[1], dtype=torch.uint8, device=dev)

    def chunked():
        for i, a in enumerate(bounds[:-1]):
            msa.msa_prefill_chunk(cq[i], cqi[i], pin["k"], pin["v"], pin["k_idx"], ckeys, a, w.block_size, w.top_k,
                                  out=couts[i], workspace=cws)

    ms = _median_ms(chunked, 5)
    res["prefill_32k_chunked"] = {"what": "the 32K prefill as four chunks of 8192 queries against the cache",
                                  "ms": round(ms, 4), "tokens_per_s": round(w.seq_len / (ms * 1e-3), 1),
                                  "tflops_alg": round(_flop_alg(w) / (ms * 1e-3) / 1e12, 2)}
    del pin, cq, cqi, couts, cws
    ws_ = get_workload("prefill_32k", top_k=32)
    Ss = 4096
    sin = prefill_inputs(ws_, seed=1, device=dev, seq_len=Ss)
    sout = torch.empty_like(sin["q"])
    skeys = torch.empty((1, ws_.n_kv_heads, Ss // ws_.block_size, 64), dtype=torch.int8, device=dev)
    sdims = msa.make_dims(1, Ss, ws_.n_q_heads, ws_.n_kv_heads, ws_.block_size, ws_.top_k)
    sws = torch.empty(msa.msa_prefill_chunk_workspace_bytes(sdims, Ss)[1], dtype=torch.uint8, device=dev)
    dense_ms = _median_ms(lambda: msa.msa_prefill(sin["q"], sin["k"], sin["v"], sin["q_idx"], sin["k_idx"],
                                                  ws_.block_size, ws_.top_k, out=sout), 5)
    sparse_ms = _median_ms(lambda: msa.msa_prefill_chunk(sin["q"], sin["q_idx"], sin["k"], sin["v"], sin["k_idx"],
                                                         skeys, 0, ws_.block_size, ws_.top_k, out=sout,
                                                         workspace=sws), 5)
    flop = 4.0 * D_HEAD * ws_.n_q_heads * Ss * (Ss + 1) / 2
    res["prefill_short_dense"] = {
        "what": "4096 tokens, top_k 32 = every block: dense causal kernel vs the sparse path on the same data",
        "dense_ms": round(dense_ms, 4), "sparse_path_ms": round(sparse_ms, 4),
        "dense_tflops": round(flop / (dense_ms * 1e-3) / 1e12, 2),
        "dense_frac_bf16_peak": round(flop / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del sin, sout, sws
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ main

def machine_probes(msa, dev):
    """What the chip sustains under plain load, beside its published peaks
    (which stay the roofline's `peak`): the library's matrix-core probe, a
    kernel of bf16 MFMAs on register operands only, and a 2 GiB device copy
    (torch's copy kernel; bytes read plus bytes written)."""
    import torch
    nwg, iters = 2048, 20000  # 8 workgroups of 4 waves per CU; about 9 ms at the published peak
    buf = torch.empty(nwg * 256, dtype=torch.float32, device=dev)
    flop = [0.0]

    def probe():
        flop[0] = msa.msa_probe_mfma_bf16(nwg, iters, buf)

    mfma_ms = _median_ms(probe, 5)
    finite = bool(torch.isfinite(buf).all())
    src = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_ms = _median_ms(lambda: dst.copy_(src), 5)
    del src, dst, buf
    torch.cuda.empty_cache()
    mfma_tflops = flop[0] / (mfma_ms * 1e-3) / 1e12
    copy_gbs = 2 * (1 << 31) / (copy_ms * 1e-3) / 1e9
    return {
        "mfma_bf16_probe_tflops": round(mfma_tflops, 1),
        "mfma_bf16_probe_frac_of_published": round(mfma_tflops / PEAK_BF16_TFLOPS, 4),
        "mfma_probe_what": f"msa_probe_mfma_bf16: {nwg} workgroups x 4 waves x {iters} rounds of 4 independent "
                           f"v_mfma_f32_32x32x16_bf16, register operands only, median of 5 launches"
                           + ("" if finite else " (non-finite output)"),
        "hbm_copy_gbs": round(copy_gbs, 1),
        "hbm_copy_frac_of_published": round(copy_gbs / PEAK_HBM_GBS, 4),
        "hbm_copy_what": "2 GiB device-to-device copy (torch), read + written bytes, median of 5",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--core-only", action="store_true",
                    help="time the step only (no other workloads, extras or CPU baseline), e.g. under a profiler")
    ap.add_argument("--prefill-workload", default=HEADLINE,
                    help="prefill workload of the step (default: the 1M prefill); another one is for profiler runs "
                         "with --core-only")
    ap.add_argument("--train-only", action="store_true",
                    help="time only the training forward (with log-sum-exp) and backward of the 32K prefill")
    ap.add_argument("--pmc-run", action="store_true",
                    help="run the counter-collection workload instead of the benchmark")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record from the two counter runs' CSV files")
    ap.add_argument("--pmc-commands", nargs="*", default=[], help=argparse.SUPPRESS)
    ap.add_argument("--counter-table", nargs="+", metavar=("STATS_CSV", "PMC_CSV"),
                    help="print the SQ counter table of the MSA kernels from a kernel-trace stats CSV and the "
                         "counter passes' CSV files")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.pmc_commands)
        return 0
    if args.counter_table:
        counter_table(args.counter_table[0], args.counter_table[1:])
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the MSA path here runs on a single MI355X; it would shard by GQA group, with no exchange).",
              file=sys.stderr)
        return 2
    if args.pmc_run:
        pmc_run()
        return 0
    if args.train_only:
        train_only(args.steps, args.warmup)
        return 0

    import torch
    import block_sparse_attention_33_amd as msa
    from synth import decode_inputs, get_workload, prefill_inputs, sample_rows

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    headline = args.prefill_workload
    wp = get_workload(headline)
    wd = get_workload(DECODE)
    _say("generating inputs")
    pin = prefill_inputs(wp, seed=0, device=dev)
    din = decode_inputs(wd, seed=0, device=dev)
    block_keys = msa.msa_pool_block_keys(din["k_idx_cache"], wd.block_size)
    out = torch.empty_like(pin["q"])
    sel = torch.empty((wp.batch, wp.n_kv_heads, wp.seq_len, wp.top_k), dtype=torch.int32, device=dev)
    dout = torch.empty_like(din["q"])
    dsel = torch.empty((wd.batch, wd.n_kv_heads, wd.top_k), dtype=torch.int32, device=dev)
    pws = _workspace(msa, msa.MSA_OP_PREFILL, wp, dev)
    dws = _workspace(msa, msa.MSA_OP_DECODE, wd, dev)

    def prefill():
        msa.msa_prefill(pin["q"], pin["k"], pin["v"], pin["q_idx"], pin["k_idx"], wp.block_size, wp.top_k, out=out,
                        sel=sel, workspace=pws)

    def decode():
        msa.msa_decode(din["q"], din["q_idx"], din["k_cache"], din["v_cache"], block_keys, wd.block_size, wd.top_k,
                       out=dout, sel=dsel, workspace=dws)

    _say(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    # Timed region: the library's kernel timing (HIP events around each of its
    # launches, on its stream) is on for the prefill (its launches are long;
    # the events cost microseconds) and off for the decode, whose kernel
    # breakdown comes from a separate pass below.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    msa.profile_read()
    torch.cuda.synchronize()
    _say(f"timing {args.steps} steps")
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
    msa.profile_enable(True)
    for _ in range(args.steps):
        decode()
    torch.cuda.synchronize()
    msa.profile_enable(False)
    dkt = msa.profile_read()

    per_head_keys, per_head_earlier, pairs = _prefill_counts(wp)
    D = wp.head_dim
    flop_alg = 4.0 * D * wp.n_q_heads * per_head_keys
    flop_att = 4.0 * D * wp.n_q_heads * per_head_earlier   # the attention kernel's share
    tokens = wp.batch * wp.seq_len
    rows = tokens * wp.n_q_heads
    # dominant kernel: the attention kernel (all kept blocks of every query),
    # one launch per query chunk
    n_att, att_ms = kt.get("attend", (0, 0.0))
    att_ms_step = att_ms / args.steps
    att_launch_ms = att_ms / max(1, n_att)
    launches_per_step = max(1, n_att // args.steps)
    att_tflops = flop_att / (att_ms_step * 1e-3) / 1e12 if att_ms_step > 0 else None
    # bytes the KV-outer design moves: per (query row, earlier kept block)
    # pair a gathered Q row (256 B) and a bf16 partial + fp32 (max, sum)
    # (264 B); the merge reads the partials back and, per row, Q (256 B) for
    # the own block and writes O (256 B) (the own blocks' K and V, 64 KB per
    # 1024 rows at the headline's shape, come mostly from L2 and are left out)
    att_design_bytes = pairs * (2 * D + 2 * D + 8)
    n_mrg, mrg_ms = kt.get("merge", (0, 0.0))
    mrg_ms_step = mrg_ms / args.steps
    mrg_design_bytes = pairs * (2 * D + 8) + rows * (2 * D + 2 * D)
    dbytes = _decode_bytes(wd)
    traffic = _measured_traffic() if headline == HEADLINE else None

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
        "config": {"workload": f"{headline} + {DECODE}", "batch": wp.batch, "seq_len": wp.seq_len,
                   "n_q_heads": wp.n_q_heads, "n_kv_heads": wp.n_kv_heads, "head_dim": D,
                   "block_size": wp.block_size, "top_k": wp.top_k, "decode_batch": wd.batch,
                   "decode_cache_len": wd.seq_len, "parallelism": "none (1 GPU)"},
        "prefill": {
            "workload": headline,
            "ms": round(pre_med, 4),
            "tokens_per_s": round(tokens / (pre_med * 1e-3), 1),
            "tflops_alg": round(flop_alg / (pre_med * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(flop_alg / (pre_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "flop_alg": flop_alg,
        },
        "decode": {
            "workload": DECODE,
            "us": round(dec_med * 1e3, 2),
            "tokens_per_s": round(wd.batch / (dec_med * 1e-3), 1),
            "hbm_gbs_alg": round(dbytes / (dec_med * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(dbytes / (dec_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_alg": dbytes,
            "timing": "right after the 1M prefill in the same stream",
        },
        "roofline": {
            "kernel": "attend_kernel<128, true> (KV-outer block attention over the kept blocks before each "
                      "query's own, one query chunk; the instance taking runs of items from a counter, used at 1M)",
            "workload": headline,
            "bound": "mfma",
            "achieved": round(att_tflops, 2) if att_tflops else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4) if att_tflops else None,
            "traffic": traffic,
            "avg_launch_ms": round(att_launch_ms, 4),
            "launches_per_step": launches_per_step,
            "flop_per_launch": flop_att / launches_per_step,
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
            "what": "own block's causal attention + log-sum-exp merge of every row's partials",
            "ms_per_step": round(mrg_ms_step, 4),
            "own_block_flop": flop_alg - flop_att,
            "design_bytes": mrg_design_bytes,
            "hbm_gbs": round(mrg_design_bytes / (mrg_ms_step * 1e-3) / 1e9, 1) if mrg_ms_step else None,
        },
        "kernels": {k: {"launches": n, "avg_ms": round(ms / max(1, n), 4)}
                    for k, (n, ms) in sorted(list(kt.items()) + list(dkt.items()))},
    }
    cpu = not (args.no_cpu_baseline or args.core_only) and headline == HEADLINE
    if headline != HEADLINE and not args.core_only:
        raise SystemExit("--prefill-workload other than the 1M prefill is for --core-only profiler runs")
    baselines = {}
    if cpu:
        _say(f"cpu baseline: {HEADLINE} ({CPU_SAMPLE_ROWS} rows), {DECODE}")
        rows = sample_rows(wp.seq_len, CPU_SAMPLE_ROWS, 12345)
        baselines[HEADLINE] = cpu_baseline_prefill(HEADLINE, pin, out, sel, rows)
        baselines[DECODE] = cpu_baseline_decode(din, block_keys, dout, dsel, wd)
    if not args.core_only:
        rec["decode"].update(decode_extras(msa, din, block_keys, wd, dws, dout, args.steps))
    del pin, out, sel, pws, din, block_keys, dout, dsel, dws
    torch.cuda.empty_cache()
    if not args.core_only:
        rec["prefill_other_workloads"], more = other_prefills(msa, dev, cpu)
        baselines.update(more)
        rec.update(chunked_and_dense(msa, dev))
        rec["training"] = training_extras(msa, dev)
        rec["machine"] = machine_probes(msa, dev)
        ach = rec["roofline"].get("achieved")
        probe = rec["machine"]["mfma_bf16_probe_tflops"]
        rec["roofline"]["probe_peak"] = probe
        rec["roofline"]["frac_of_probe"] = round(ach / probe, 4) if (ach and probe) else None
    rec["cpu_baseline"] = baselines.get(HEADLINE)
    rec["cpu_baselines"] = baselines or None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
