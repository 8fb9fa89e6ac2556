"""The CPU oracle over many query rows at once, in worker processes --
TEST INFRASTRUCTURE ONLY (the test suite and the benchmark's CPU-baseline
leg use it; the library never does).

The oracle is single-threaded by design; full-size parity checks (every row
of a 32K prefill, 4096 sampled rows of the 128K and 1M prefills, the query
gradients of hundreds of sampled rows) run it over thousands of rows, so the rows are split over fresh worker processes
("spawn": they start from nothing, import only numpy and the oracle, and
never touch the GPU).  Inputs reach them as memory-mapped .npy files in a
temporary directory (bf16 tensors as their 16-bit patterns, widened to
float32 exactly on access); each worker writes its rows' selection and
bf16-rounded output straight into shared output files.

This module holds none of the method's arithmetic: every value comes from
oracle/msa_oracle.py.
"""
import os
import shutil
import tempfile
import time

import numpy as np

from oracle import msa_oracle as O

MAX_WORKERS = 12


class Bf16Bits:
    """Read-only view of bf16 values stored as uint16 bit patterns; indexing
    returns the float32 values (exact: bf16 is the top half of float32)."""

    def __init__(self, bits: np.ndarray):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return (np.asarray(self.bits[idx]).astype(np.uint32) << 16).view(np.float32)


def n_workers() -> int:
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, avail))


def _scratch_dir() -> str:
    """A temporary directory, in RAM-backed /dev/shm when it has room."""
    base = None
    try:
        if os.path.isdir("/dev/shm") and shutil.disk_usage("/dev/shm").free > (48 << 30):
            base = "/dev/shm"
    except OSError:
        base = None
    return tempfile.mkdtemp(prefix="msa_oracle_", dir=base)


def _map(worker, jobs, n):
    """worker(job) for every job, in up to n fresh one-thread processes that
    never touch the GPU; returns the sum of the workers' results."""
    if n == 1 or len(jobs) == 1:
        return sum(worker(j) for j in jobs)
    import concurrent.futures as cf
    import multiprocessing as mp
    keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS",
                                           "HIP_VISIBLE_DEVICES", "CUDA_VISIBLE_DEVICES")}
    os.environ.update(OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
                      HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    try:
        # an executor, not a Pool: a worker that dies (e.g. cannot import its
        # module) fails the call instead of being respawned
        with cf.ProcessPoolExecutor(max_workers=min(n, len(jobs)), mp_context=mp.get_context("spawn")) as ex:
            return sum(ex.map(worker, jobs))
    finally:
        for k, val in keep.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val


def _prefill_worker(job):
    d, lo, hi, bs, top_k, scale = job
    ld = lambda name: np.load(os.path.join(d, name + ".npy"), mmap_mode="r")  # noqa: E731
    rows = np.asarray(ld("rows")[lo:hi])
    q_rows = Bf16Bits(ld("q_rows"))[:, lo:hi]
    k, v = Bf16Bits(ld("k")), Bf16Bits(ld("v"))
    sel = O.select_blocks(ld("q_idx"), np.asarray(ld("summ")), bs, top_k, rows)
    out = O.attention_rows(q_rows, k, v, sel, rows, bs, scale)
    osel = np.load(os.path.join(d, "out_sel.npy"), mmap_mode="r+")
    oout = np.load(os.path.join(d, "out_o.npy"), mmap_mode="r+")
    osel[:, :, lo:hi] = sel
    oout[:, lo:hi] = O.round_to_bf16(out).astype(np.float32)
    osel.flush()
    oout.flush()
    return hi - lo


def prefill_rows(q_bits, k_bits, v_bits, q_idx, k_idx, rows, block_size, top_k, scale=None, workers=None):
    """Oracle summaries, selection and bf16-rounded output for query `rows`.

    q_bits [B, R, Hq, D] uint16: the bf16 bits of the R sampled query rows;
    k_bits, v_bits [B, G, S, D] uint16; q_idx, k_idx [B, G, S, di] int8
    (numpy).  Returns (summaries int8 [B, G, nb, di], sel int32
    [B, G, R, top_k], out float32 [B, R, Hq, D] holding bf16 values, stats).
    """
    rows = np.asarray(rows, dtype=np.int64)
    B, R, Hq, D = q_bits.shape
    G = k_bits.shape[1]
    summ = O.pool_block_keys(k_idx, block_size)
    n = workers or n_workers()
    d = _scratch_dir()
    t0 = time.perf_counter()
    try:
        for name, arr in (("rows", rows), ("q_rows", q_bits), ("k", k_bits), ("v", v_bits), ("q_idx", q_idx),
                          ("summ", summ)):
            np.save(os.path.join(d, name + ".npy"), arr)
        np.lib.format.open_memmap(os.path.join(d, "out_sel.npy"), mode="w+", dtype=np.int32,
                                  shape=(B, G, R, top_k)).flush()
        np.lib.format.open_memmap(os.path.join(d, "out_o.npy"), mode="w+", dtype=np.float32,
                                  shape=(B, R, Hq, D)).flush()
        step = max(1, -(-R // (4 * n)))
        jobs = [(d, lo, min(R, lo + step), block_size, top_k, scale) for lo in range(0, R, step)]
        assert _map(_prefill_worker, jobs, n) == R
        sel = np.array(np.load(os.path.join(d, "out_sel.npy")))
        out = np.array(np.load(os.path.join(d, "out_o.npy")))
    finally:
        shutil.rmtree(d, ignore_errors=True)
    stats = {"rows": int(R), "workers": int(min(n, len(jobs))), "seconds": round(time.perf_counter() - t0, 2)}
    return summ, sel, out, stats


def _grad_worker(job):
    d, lo, hi, bs, scale = job
    ld = lambda name: np.load(os.path.join(d, name + ".npy"), mmap_mode="r")  # noqa: E731
    rows = np.asarray(ld("rows")[lo:hi])
    q_rows = Bf16Bits(ld("q_rows"))[:, lo:hi]
    do_rows = Bf16Bits(ld("do_rows"))[:, lo:hi]
    k, v = Bf16Bits(ld("k")), Bf16Bits(ld("v"))
    sel = np.asarray(ld("sel")[:, :, lo:hi])
    dq = O.query_grad_rows(q_rows, k, v, do_rows, sel, rows, bs, scale)
    out = np.load(os.path.join(d, "out_dq.npy"), mmap_mode="r+")
    out[:, lo:hi] = dq
    out.flush()
    return hi - lo


def query_grad_rows(q_bits, do_bits, k_bits, v_bits, sel, rows, block_size, scale=None, workers=None):
    """The oracle's dq (msa_oracle.query_grad_rows, float64 [B, R, Hq, D])
    of query `rows`, the rows split over worker processes.

    q_bits, do_bits [B, R, Hq, D] uint16: the bf16 bits of those rows of q
    and of the output gradient; k_bits, v_bits [B, G, S, D] uint16; sel
    int32 [B, G, R, top_k]: the rows' selections.  Returns (dq, stats)."""
    rows = np.asarray(rows, dtype=np.int64)
    B, R, Hq, D = q_bits.shape
    n = workers or n_workers()
    d = _scratch_dir()
    t0 = time.perf_counter()
    try:
        for name, arr in (("rows", rows), ("q_rows", q_bits), ("do_rows", do_bits), ("k", k_bits), ("v", v_bits),
                          ("sel", np.asarray(sel, dtype=np.int32))):
            np.save(os.path.join(d, name + ".npy"), arr)
        np.lib.format.open_memmap(os.path.join(d, "out_dq.npy"), mode="w+", dtype=np.float64,
                                  shape=(B, R, Hq, D)).flush()
        step = max(1, -(-R // (4 * n)))
        jobs = [(d, lo, min(R, lo + step), block_size, scale) for lo in range(0, R, step)]
        assert _map(_grad_worker, jobs, n) == R
        dq = np.array(np.load(os.path.join(d, "out_dq.npy")))
    finally:
        shutil.rmtree(d, ignore_errors=True)
    stats = {"rows": int(R), "workers": int(min(n, len(jobs))), "seconds": round(time.perf_counter() - t0, 2)}
    return dq, stats


def _kv_grad_worker(job):
    d, i, bs, scale = job
    ld = lambda name: np.load(os.path.join(d, name + ".npy"), mmap_mode="r")  # noqa: E731
    j, g = (int(x) for x in ld("pairs")[i])
    q, do = Bf16Bits(ld("q")), Bf16Bits(ld("dout"))
    k, v = Bf16Bits(ld("k")), Bf16Bits(ld("v"))
    _, dk, dv = O.backward(q, k, v, do, ld("sel"), bs, scale, rows=[], kv_blocks=[j], groups=[g])
    ok = np.load(os.path.join(d, "out_dk.npy"), mmap_mode="r+")
    ov = np.load(os.path.join(d, "out_dv.npy"), mmap_mode="r+")
    ok[:, i] = dk[:, g, 0]
    ov[:, i] = dv[:, g, 0]
    ok.flush()
    ov.flush()
    return 1


def kv_grad_pairs(q_bits, do_bits, k_bits, v_bits, sel, pairs, block_size, scale=None, workers=None):
    """The oracle's dk and dv (msa_oracle.backward) of key block j in group g
    for each (j, g) of `pairs`, one pair per job over worker processes (a
    pair's cost is the number of queries that kept the block).

    q_bits, do_bits [B, S, Hq, D] uint16 (bf16 bits of every query row and
    of the output gradient); k_bits, v_bits [B, G, S, D] uint16; sel int32
    [B, G, S, top_k]: every row's selection.  Returns (dk, dv float64
    [B, len(pairs), block_size, D], stats); rows of a ragged last block past
    the sequence end stay zero."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    B, S, Hq, D = q_bits.shape
    P = len(pairs)
    n = workers or n_workers()
    d = _scratch_dir()
    t0 = time.perf_counter()
    try:
        for name, arr in (("pairs", pairs), ("q", q_bits), ("dout", do_bits), ("k", k_bits), ("v", v_bits),
                          ("sel", np.asarray(sel, dtype=np.int32))):
            np.save(os.path.join(d, name + ".npy"), arr)
        for name in ("out_dk", "out_dv"):
            np.lib.format.open_memmap(os.path.join(d, name + ".npy"), mode="w+", dtype=np.float64,
                                      shape=(B, P, block_size, D)).flush()
        jobs = [(d, i, block_size, scale) for i in range(P)]
        assert _map(_kv_grad_worker, jobs, n) == P
        dk = np.array(np.load(os.path.join(d, "out_dk.npy")))
        dv = np.array(np.load(os.path.join(d, "out_dv.npy")))
    finally:
        shutil.rmtree(d, ignore_errors=True)
    stats = {"pairs": int(P), "workers": int(min(n, P)), "seconds": round(time.perf_counter() - t0, 2)}
    return dk, dv, stats
