"""Shared helpers of the GPU parity tests: host copies of device inputs for
the oracle and the output comparison."""
import json
import os
import sys

import numpy as np
import torch

from oracle import msa_oracle as O

MAX_ABS = 1e-2     # max |gpu - bf16(oracle)| over compared elements
MEAN_ABS = 1e-3    # mean |gpu - bf16(oracle)| over compared elements
# Scale-relative bar, per compared (row, head): the mean error of the head's
# 128 outputs against the mean |bf16(oracle)| of those outputs.  Rounding
# the output to bf16 alone gives 0.14-0.18 % (32K workload, exact attention
# rounded); the GPU adds bf16 P as an MFMA operand and bf16 partials, a few
# times that.  Dropping one of a row's kept blocks moves it by 11 % at the
# least and 25 % at the median (same workload, 200 rows x 8 groups, one
# random non-own block removed, computed with the oracle).  The bar sits
# between, so that a mistake confined to a few rows cannot hide under the
# absolute bar, which is a third of the typical output at 32K tokens.  (The
# largest error of a (row, head) against its mean magnitude is printed as
# well: it is dominated by bf16 steps of the largest outputs, about 1.6 %
# per step, so it is reported, not barred.)
ROW_REL_MAX = 0.03

STATS_FILE = os.environ.get("MSA_PARITY_STATS")   # optional JSON-lines record of every comparison


def host_f32(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> float32 numpy (exact)."""
    return t.detach().to("cpu").float().numpy()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> its 16-bit patterns as uint16 numpy."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


class HostBf16:
    """A host copy of a bf16 tensor, kept as 16-bit patterns, that hands out
    float32 numpy slices (exact), so the oracle can gather rows of a large
    cache without a full fp32 copy."""

    def __init__(self, t: torch.Tensor):
        self.bits = host_bits(t)
        self.shape = tuple(self.bits.shape)

    def __getitem__(self, idx):
        return (np.asarray(self.bits[idx]).astype(np.uint32) << 16).view(np.float32)


def host_i8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").numpy()


def record(what, rec):
    """Print one comparison's observed errors (and append them to the
    MSA_PARITY_STATS file when that is set)."""
    line = json.dumps({"what": what, **rec})
    print(f"[parity] {line}", flush=True)
    sys.stdout.flush()
    if STATS_FILE:
        with open(STATS_FILE, "a") as f:
            f.write(line + "\n")


def compare_rounded(gpu_bf16: torch.Tensor, ref_bf16: np.ndarray, what: str):
    """Compare a GPU bf16 output [..., Hq, D] with the oracle already rounded
    to bf16: absolute bars over every element and the per-(row, head)
    scale-relative bar.  Prints (and optionally records) the observed
    errors; returns them."""
    g = host_f32(gpu_bf16).astype(np.float64)
    ref = np.asarray(ref_bf16, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    d = np.abs(g - ref)
    max_abs, mean_abs = float(d.max()), float(d.mean())
    scale = np.maximum(np.abs(ref).mean(axis=-1), 1e-30)
    ratio = d.mean(axis=-1) / scale
    peak = d.max(axis=-1) / scale
    worst = np.unravel_index(int(ratio.argmax()), ratio.shape)
    rec = {"elements": int(d.size), "max_abs": max_abs, "mean_abs": mean_abs,
           "mean_abs_oracle": float(np.abs(ref).mean()), "max_row_rel": float(ratio.max()),
           "median_row_rel": float(np.median(ratio)), "max_row_peak_rel": float(peak.max()),
           "bars": [MAX_ABS, MEAN_ABS, ROW_REL_MAX]}
    record(what, rec)
    assert max_abs <= MAX_ABS and mean_abs <= MEAN_ABS, (
        f"{what}: max_abs={max_abs:.3e} (<= {MAX_ABS}), mean_abs={mean_abs:.3e} (<= {MEAN_ABS}), "
        f"worst at {np.unravel_index(int(d.argmax()), d.shape)}")
    assert float(ratio.max()) <= ROW_REL_MAX, (
        f"{what}: a (row, head) mean error {ratio.max():.3e} of its mean |output| (<= {ROW_REL_MAX}) at {worst}")
    return rec


def compare_out(gpu_bf16: torch.Tensor, oracle_f64: np.ndarray, what: str):
    """Compare a GPU bf16 output with the oracle's fp64 result rounded to bf16."""
    rec = compare_rounded(gpu_bf16, O.round_to_bf16(oracle_f64), what)
    return rec["max_abs"], rec["mean_abs"]


def oracle_prefill_rows(inp, w, rows, block_size=None, top_k=None):
    """Oracle summaries, selection and output for the given rows, from host
    copies of the device inputs."""
    bs = block_size or w.block_size
    k = top_k or w.top_k
    q_rows = host_f32(inp["q"][:, torch.as_tensor(rows, device=inp["q"].device)])
    kk = HostBf16(inp["k"])
    vv = HostBf16(inp["v"])
    qi = host_i8(inp["q_idx"])
    ki = host_i8(inp["k_idx"])
    summ = O.pool_block_keys(ki, bs)
    sel = O.select_blocks(qi, summ, bs, k, rows)
    out = O.attention_rows(q_rows, kk, vv, sel, rows, bs)
    return summ, sel, out


def oracle_prefill_rows_pooled(inp, w, rows, block_size=None, top_k=None):
    """The same for many rows, over worker processes: (summaries, sel,
    bf16-rounded output as float32, stats)."""
    from oracle import pool as oracle_pool
    bs = block_size or w.block_size
    k = top_k or w.top_k
    rt = torch.as_tensor(rows, device=inp["q"].device)
    return oracle_pool.prefill_rows(host_bits(inp["q"][:, rt]), host_bits(inp["k"]), host_bits(inp["v"]),
                                    host_i8(inp["q_idx"]), host_i8(inp["k_idx"]), rows, bs, k)


def oracle_query_grads_pooled(inp, dout, sel_rows, rows, block_size):
    """The oracle's dq of query `rows` (float64 [B, R, Hq, D]) over worker
    processes, from host copies of the device inputs; sel_rows int32
    [B, G, R, top_k] are the rows' (oracle) selections.  Returns (dq, stats)."""
    from oracle import pool as oracle_pool
    rt = torch.as_tensor(rows, device=inp["q"].device)
    return oracle_pool.query_grad_rows(host_bits(inp["q"][:, rt]), host_bits(dout[:, rt]), host_bits(inp["k"]),
                                       host_bits(inp["v"]), sel_rows, rows, block_size)


def oracle_kv_grads_pooled(inp, dout, sel, pairs, block_size):
    """The oracle's dk, dv (float64 [B, P, block_size, D]) of key block j in
    group g for each (j, g) of `pairs`, over worker processes; sel int32
    [B, G, S, top_k] is every row's (oracle) selection.  Returns (dk, dv,
    stats)."""
    from oracle import pool as oracle_pool
    return oracle_pool.kv_grad_pairs(host_bits(inp["q"]), host_bits(dout), host_bits(inp["k"]), host_bits(inp["v"]),
                                     sel, pairs, block_size)


def check_all_selections(gsel, qi, summ, S, bs, top_k, row_slice=8192, rows=None):
    """Every row of `rows` (default all): with the composite key score * 2^20
    - block (higher is better, ties to the lower block), the kept set is
    exactly the top min(top_k - 1, own) of the earlier blocks, and the own
    block follows.  gsel [1, G, S, top_k], qi [1, G, S, di] (int), summ
    [1, G, nb, di].  Scores are exact integer dot products computed with
    float64 BLAS: every product (|.| <= 2^14) and partial sum (|.| <= 2^20)
    is an integer far below 2^53, so no rounding occurs."""
    kp = top_k - 1
    nb = summ.shape[2]
    j = np.arange(nb)[None, :]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    for g in range(summ.shape[1]):
        sf = summ[0, g].astype(np.float64)
        for r0 in range(0, len(rows), row_slice):
            rr = rows[r0:r0 + row_slice]
            own = rr // bs
            sc = qi[0, g, rr].astype(np.float64) @ sf.T                      # [n, nb], exact integers
            key = sc * float(1 << 20) - j
            valid = j < own[:, None]
            key = np.where(valid, key, -np.inf)
            if kp > 0:
                thr = -np.partition(-key, kp - 1, axis=1)[:, kp - 1]
            else:
                thr = np.full(len(rr), np.inf)
            expect = (key >= thr[:, None]) & valid
            kept = np.asarray(gsel[0, g, rr])
            got = np.zeros((len(rr), nb), bool)
            ri, ci = np.nonzero(kept >= 0)
            got[ri, kept[ri, ci]] = True
            got[np.arange(len(rr)), own] = False
            assert np.array_equal(got, expect), f"group {g}, rows {rr[0]}..{rr[-1]}"
            m = np.minimum(kp, own)
            assert (kept[np.arange(len(rr)), m] == own).all(), f"group {g}: own block not after the kept ones"
            assert (np.where(np.arange(top_k)[None, :] > m[:, None], kept, -1) == -1).all(), "padding"
