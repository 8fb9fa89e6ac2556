"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Selections and block summaries must match bit for bit; outputs must be
within max-abs 1e-2 and mean-abs 1e-3 of the oracle's fp64 result rounded to
bf16, and every compared (row, head) with a mean error within 3 % of its own
mean magnitude (tests/helpers.py).  Small cases compare every row; at full size the 32K
prefill compares every row, the structured 128K and the 1M prefills 32768
seeded rows each (the oracle runs over worker processes), and the 128K
selections and three ranges of 16384 rows of the 1M index (the first, the
middle and the last) are checked in full.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_33_amd as msa
from oracle import msa_oracle as O
from synth import decode_inputs, get_workload, prefill_inputs, sample_rows
from tests.helpers import (HostBf16, check_all_selections, compare_out, compare_rounded, host_f32, host_i8,
                           oracle_prefill_rows, oracle_prefill_rows_pooled)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _run_prefill(inp, bs, k, **kw):
    out, sel = msa.msa_prefill(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], bs, k,
                               return_sel=True, **kw)
    torch.cuda.synchronize()
    return out, sel


# ------------------------------------------------------------------ small cases, all rows

SMALL = [
    # name, workload overrides, seq_len
    ("tiny_2k", {}, None),
    ("ragged_gqa4", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=5), 1000),
    ("batch2_r1_bs32", dict(batch=2, n_q_heads=2, n_kv_heads=2, block_size=32, top_k=4), 600),
    ("r16_bs128", dict(n_q_heads=16, n_kv_heads=1, block_size=128, top_k=3), 777),
    ("topk1_own_only", dict(n_q_heads=8, n_kv_heads=1, top_k=1), 700),
    ("topk_ge_nb_dense", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=32), 1100),
    ("single_block", dict(n_q_heads=8, n_kv_heads=1, block_size=128, top_k=4), 100),
    ("r2_bs64_k2", dict(n_q_heads=4, n_kv_heads=2, block_size=64, top_k=2), 513),
    ("one_token", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=4), 1),
    ("three_tokens_b3_r1", dict(batch=3, n_q_heads=2, n_kv_heads=2, block_size=32, top_k=2), 3),
]


@pytest.mark.parametrize("name,over,S", SMALL, ids=[c[0] for c in SMALL])
def test_prefill_small_all_rows(name, over, S):
    w = get_workload("tiny_2k", **over)
    _say(f"[prefill small] {name} S={S or w.seq_len} {w}")
    inp = prefill_inputs(w, seed=11, device="cpu", seq_len=S)
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    out, sel = _run_prefill(dinp, w.block_size, w.top_k)
    rows = np.arange(inp["q"].shape[1])
    summ, osel, oout = oracle_prefill_rows(inp, w, rows)
    assert np.array_equal(host_i8(sel).astype(np.int32), osel), f"{name}: selection differs"
    compare_out(out, oout, name)


def test_index_select_bit_exact():
    w = get_workload("tiny_2k", n_q_heads=8, n_kv_heads=4, top_k=6)
    _say("[index_select] S=4096 G=4 k=6")
    inp = prefill_inputs(w, seed=3, device="cpu", seq_len=4096)
    bk, sel = msa.msa_index_select(inp["q_idx"].to(DEV), inp["k_idx"].to(DEV), w.block_size, w.top_k)
    torch.cuda.synchronize()
    summ = O.pool_block_keys(inp["k_idx"].numpy(), w.block_size)
    assert np.array_equal(host_i8(bk), summ)
    osel = O.select_blocks(inp["q_idx"].numpy(), summ, w.block_size, w.top_k)
    assert np.array_equal(host_i8(sel).astype(np.int32), osel)


def test_pool_negative_means_floor():
    # every block alternates -1 / 0: the floor of the mean is -1 (truncation gives 0)
    k_idx = torch.zeros((1, 2, 256, 64), dtype=torch.int8)
    k_idx[:, :, 0::2] = -1
    _say("[pool] floor of negative means")
    bk = msa.msa_pool_block_keys(k_idx.to(DEV), 64)
    torch.cuda.synchronize()
    assert (host_i8(bk) == -1).all()


@pytest.mark.parametrize("S,top_k", [(2048, 9), (8192, 16), (12000, 32)])
def test_index_ties_go_to_lower_block(S, top_k):
    """Index values in {-1, 0, 1}: summaries are mostly -1/0 and many scores
    tie.  2048 tokens in 32-token blocks rank at most 63 blocks (one LDS
    chunk of summaries); 8192 and 12000 tokens rank up to 255 and 374 blocks,
    so the matrix-core top-k crosses summary chunks with tied scores on both
    sides of the chunk boundaries and of its half-list merge.  Every row
    against the oracle."""
    g = torch.Generator().manual_seed(5 + S)
    q_idx = torch.randint(-1, 2, (1, 2, S, 64), generator=g, dtype=torch.int8)
    k_idx = torch.randint(-1, 2, (1, 2, S, 64), generator=g, dtype=torch.int8)
    _say(f"[index] ties S={S} top_k={top_k}")
    bk, sel = msa.msa_index_select(q_idx.to(DEV), k_idx.to(DEV), 32, top_k)
    torch.cuda.synchronize()
    summ = O.pool_block_keys(k_idx.numpy(), 32)
    assert np.array_equal(host_i8(bk), summ)
    gsel = host_i8(sel).astype(np.int32)
    rows = sample_rows(S, 1024, S)
    osel = O.select_blocks(q_idx.numpy(), summ, 32, top_k, rows)
    assert np.array_equal(gsel[:, :, rows], osel)
    check_all_selections(gsel, q_idx.numpy(), summ, S, 32, top_k)


def test_first_row_is_first_value():
    w = get_workload("tiny_2k")
    inp = prefill_inputs(w, seed=8, device=DEV, seq_len=256)
    _say("[prefill] t=0 returns v_0")
    out, _ = _run_prefill(inp, w.block_size, w.top_k)
    v0 = inp["v"][0, 0, 0]
    for h in range(w.n_q_heads):
        assert torch.equal(out[0, 0, h], v0)


def test_prefill_deterministic_and_pass_count_invariant():
    w = get_workload("prefill_32k")
    S = 8192
    _say(f"[prefill] determinism / passes S={S}")
    inp = prefill_inputs(w, seed=2, device=DEV, seq_len=S)
    dims = msa.make_dims(1, S, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
    lo, hi = msa.msa_workspace_bytes(msa.MSA_OP_PREFILL, dims)
    ws_full = torch.empty(hi, dtype=torch.uint8, device=DEV)
    a, sa = _run_prefill(inp, w.block_size, w.top_k, workspace=ws_full)
    b, sb = _run_prefill(inp, w.block_size, w.top_k, workspace=ws_full)
    del ws_full
    ws_min = torch.empty(lo, dtype=torch.uint8, device=DEV)
    c, sc = _run_prefill(inp, w.block_size, w.top_k, workspace=ws_min)
    assert torch.equal(sa, sb) and torch.equal(sa, sc)
    assert torch.equal(a, b) and torch.equal(a, c)


def test_prefill_invariants():
    w = get_workload("prefill_32k")
    S = 16384
    _say(f"[prefill] selection invariants S={S}")
    inp = prefill_inputs(w, seed=4, device=DEV, seq_len=S)
    _, sel = _run_prefill(inp, w.block_size, w.top_k)
    s = sel.long()
    own = (torch.arange(S, device=DEV) // w.block_size)
    valid = s >= 0
    # own block present and last among the valid entries
    nval = valid.sum(-1)
    last = torch.gather(s, -1, (nval - 1).unsqueeze(-1)).squeeze(-1)
    assert torch.equal(last, own.expand_as(last))
    # strictly ascending valid entries, padding only at the end
    d = s[..., 1:] - s[..., :-1]
    assert bool(((d > 0) | ~valid[..., 1:]).all())
    assert bool((valid[..., :-1] | ~valid[..., 1:]).all())
    # count = min(top_k - 1, own) + 1
    assert torch.equal(nval, torch.clamp(own, max=w.top_k - 1).expand_as(nval) + 1)


# ------------------------------------------------------------------ full-size workloads, sampled rows

def _full_prefill_case(name, n_rows, seed, ws_cap_gb=None, all_selections=False):
    """The workload's prefill on the GPU; selection and output of n_rows
    seeded rows (all rows when n_rows >= S) against the oracle, and, with
    all_selections, every row's selection against the exact top-k rule."""
    w = get_workload(name)
    _say(f"[prefill full] {name} S={w.seq_len} compared rows={min(n_rows, w.seq_len)}")
    inp = prefill_inputs(w, seed=seed, device=DEV)
    kw = {}
    if ws_cap_gb is not None:
        dims = msa.make_dims(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
        lo, hi = msa.msa_workspace_bytes(msa.MSA_OP_PREFILL, dims)
        size = int(min(hi, max(lo, ws_cap_gb * 2**30)))
        kw["workspace"] = torch.empty(size, dtype=torch.uint8, device=DEV)
    out, sel = _run_prefill(inp, w.block_size, w.top_k, **kw)
    kw.clear()
    _free()
    rows = sample_rows(w.seq_len, n_rows, seed)
    rows_t = torch.as_tensor(rows, device=DEV)
    gsel = host_i8(sel[:, :, rows_t]).astype(np.int32)
    gout = out[:, rows_t]
    _say(f"[prefill full] {name}: oracle on {len(rows)} rows")
    summ, osel, oout, st = oracle_prefill_rows_pooled(inp, w, rows)
    _say(f"[prefill full] {name}: oracle {st}")
    assert np.array_equal(gsel, osel), f"{name}: selection differs on compared rows"
    compare_rounded(gout, oout, f"{name} ({len(rows)} rows)")
    del gout, oout
    if all_selections:
        _say(f"[prefill full] {name}: every row's selection")
        check_all_selections(host_i8(sel), host_i8(inp["q_idx"]), summ, w.seq_len, w.block_size, w.top_k)
    del inp, out, sel
    _free()


def test_prefill_32k_all_rows():
    _full_prefill_case("prefill_32k", 1 << 30, seed=21)


def test_prefill_32k_selection_all_rows():
    w = get_workload("prefill_32k")
    _say("[index full] prefill_32k all rows")
    inp = prefill_inputs(w, seed=21, device=DEV)
    bk, sel = msa.msa_index_select(inp["q_idx"], inp["k_idx"], w.block_size, w.top_k)
    torch.cuda.synchronize()
    summ = O.pool_block_keys(host_i8(inp["k_idx"]), w.block_size)
    assert np.array_equal(host_i8(bk), summ)
    # vectorised check of every row: scores from the oracle's summaries, the
    # kept set must be exactly the best top_k - 1 by (score desc, index asc)
    qi = host_i8(inp["q_idx"]).astype(np.int64)
    gsel = host_i8(sel).astype(np.int64)
    S, bs = w.seq_len, w.block_size
    rows = sample_rows(S, 2048, 99)
    osel = O.select_blocks(host_i8(inp["q_idx"]), summ, bs, w.top_k, rows)
    assert np.array_equal(gsel[:, :, rows], osel)
    check_all_selections(gsel, qi, summ, S, bs, w.top_k)


@pytest.mark.parametrize("S,top_k,B", [(40000, 12, 1), (20000, 32, 1), (20000, 2, 2), (17000, 5, 1), (9000, 1, 1)])
def test_index_select_many_blocks_all_rows(S, top_k, B):
    """Thousands of tokens in blocks of 32 (531 to 1250 blocks): the queries
    rank enough blocks for the matrix-core scoring; every selection is
    checked, and sampled rows against the oracle's selection."""
    w = get_workload("tiny_2k", batch=B, n_q_heads=4, n_kv_heads=2, block_size=32, top_k=top_k)
    _say(f"[index many blocks] S={S} bs=32 k={top_k} B={B}")
    inp = prefill_inputs(w, seed=77 + top_k, device=DEV, seq_len=S)
    bk, sel = msa.msa_index_select(inp["q_idx"], inp["k_idx"], w.block_size, w.top_k)
    torch.cuda.synchronize()
    summ = O.pool_block_keys(host_i8(inp["k_idx"]), w.block_size)
    assert np.array_equal(host_i8(bk), summ)
    gsel = host_i8(sel).astype(np.int64)
    rows = sample_rows(S, 512, 77)
    osel = O.select_blocks(host_i8(inp["q_idx"]), summ, w.block_size, w.top_k, rows)
    assert np.array_equal(gsel[:, :, rows], osel)
    qi = host_i8(inp["q_idx"]).astype(np.int64)
    for b in range(B):
        check_all_selections(gsel[b:b + 1], qi[b:b + 1], summ[b:b + 1], S, w.block_size, w.top_k)


@pytest.mark.parametrize("top_k", [5, 16, 32])
def test_index_select_wide_scores_all_rows(top_k):
    """Scores spread over more than 16 bits: a few planted blocks whose
    summaries align with the group's query direction score about 2^18
    while the rest stay near zero.  Queries before the first planted block
    keep the narrow rank keys; the later ones take the single-sweep path.
    Every selection is checked, sampled rows against the oracle."""
    S, bs, G, di = 24000, 32, 2, 64
    rng = np.random.default_rng(2024)
    u = rng.integers(-64, 64, size=(G, di))
    qi = np.clip(u[:, None, :] + rng.integers(-16, 16, size=(G, S, di)), -128, 127).astype(np.int8)
    ki = rng.integers(-64, 64, size=(G, S, di)).astype(np.int8)
    hot = list(range(400, S // bs, 37))
    for g in range(G):
        for j in hot:
            noise = rng.integers(-4, 4, size=(bs, di))
            ki[g, j * bs:(j + 1) * bs] = np.clip(np.sign(u[g]) * 127 + noise, -128, 127)
    _say(f"[index wide scores] S={S} bs={bs} top_k={top_k} hot blocks={len(hot)}")
    q_idx = torch.from_numpy(qi[None]).to(DEV)
    k_idx = torch.from_numpy(ki[None]).to(DEV)
    bk, sel = msa.msa_index_select(q_idx, k_idx, bs, top_k)
    torch.cuda.synchronize()
    summ = O.pool_block_keys(ki[None], bs)
    assert np.array_equal(host_i8(bk), summ)
    gsel = host_i8(sel).astype(np.int64)
    assert gsel.min() >= -1
    rows = sample_rows(S, 512, 2024)
    osel = O.select_blocks(qi[None], summ, bs, top_k, rows)
    assert np.array_equal(gsel[:, :, rows], osel)
    # the planted blocks (9 of them) are kept by every later query that
    # keeps as many
    late = np.arange((hot[-1] + 1) * bs, S)
    if top_k - 1 >= len(hot):
        for j in hot:
            assert (gsel[0, :, late] == j).any(-1).all()
    check_all_selections(gsel, qi[None].astype(np.int64), summ, S, bs, top_k)


@pytest.mark.parametrize("nb", [65000, 65625])
def test_index_select_block_index_limit(nb):
    """Either side of the two-sweep kernel's block limit (65408 blocks, so
    that its keys hold every block index below 65536): 65000 blocks of 32
    tokens rank on the two-sweep kernel, 65625 on the single-sweep one.  One
    group; the last 2048 rows against the exact top-k rule, 256 of them
    against the oracle."""
    S, bs, top_k = nb * 32, 32, 16
    g = torch.Generator().manual_seed(nb)
    q_idx = torch.randint(-64, 64, (1, 1, S, 64), generator=g, dtype=torch.int8)
    k_idx = torch.randint(-64, 64, (1, 1, S, 64), generator=g, dtype=torch.int8)
    _say(f"[index block limit] S={S} nb={nb}")
    bk, sel = msa.msa_index_select(q_idx.to(DEV), k_idx.to(DEV), bs, top_k)
    torch.cuda.synchronize()
    summ = O.pool_block_keys(k_idx.numpy(), bs)
    assert np.array_equal(host_i8(bk), summ)
    gsel = host_i8(sel)
    qi = q_idx.numpy()
    rows = np.arange(S - 2048, S)
    check_all_selections(gsel, qi, summ, S, bs, top_k, row_slice=512, rows=rows)
    some = sample_rows(2048, 256, nb) + (S - 2048)
    osel = O.select_blocks(qi, summ, bs, top_k, some)
    assert np.array_equal(gsel[:, :, some].astype(np.int32), osel)
    del bk, sel
    _free()


def test_structured_128k_sampled():
    # 32768 of the 131072 rows: every row takes the oracle about three
    # minutes over 12 worker processes
    _full_prefill_case("structured_128k", 32768, seed=31, all_selections=True)


def test_prefill_1m_sampled():
    _full_prefill_case("prefill_1m", 32768, seed=41, ws_cap_gb=70)


def test_index_1m_16k_ranges_all_selections():
    """The 1M workload's index branch alone (msa_index_select) on three
    ranges of 16384 queries: the first (fewer earlier blocks than kept
    slots up to query 1920, then 15 to 127 candidates), the middle (about
    4096 candidates in 32 summary chunks of the matrix-core top-k) and the
    last (8064 to 8191 candidates in 64 chunks).  Every row of them is
    checked against the exact top-k rule, 512 of each against the oracle."""
    w = get_workload("prefill_1m")
    S = w.seq_len
    _say(f"[index 1M] S={S}")
    inp = prefill_inputs(w, seed=43, device=DEV)
    q_idx, k_idx = inp["q_idx"], inp["k_idx"]
    del inp
    _free()
    bk, sel = msa.msa_index_select(q_idx, k_idx, w.block_size, w.top_k)
    torch.cuda.synchronize()
    summ = O.pool_block_keys(host_i8(k_idx), w.block_size)
    assert np.array_equal(host_i8(bk), summ)
    gsel = host_i8(sel)
    qi = host_i8(q_idx)
    for r0 in (0, S // 2 - 8192, S - 16384):
        _say(f"[index 1M] rows {r0} .. {r0 + 16383}")
        rows = np.arange(r0, r0 + 16384)
        check_all_selections(gsel, qi, summ, S, w.block_size, w.top_k, row_slice=2048, rows=rows)
        some = sample_rows(16384, 512, 43) + r0
        osel = O.select_blocks(qi, summ, w.block_size, w.top_k, some)
        assert np.array_equal(gsel[:, :, some].astype(np.int32), osel), f"selection differs in rows {r0}+"
    del q_idx, k_idx, bk, sel
    _free()


# ------------------------------------------------------------------ dense fallback (top_k >= nb)

DENSE = [
    # name, workload overrides, S
    ("r1_bs32_tiles_span_blocks", dict(n_q_heads=2, n_kv_heads=2, block_size=32, top_k=32), 700),
    ("r16_bs128", dict(n_q_heads=16, n_kv_heads=1, block_size=128, top_k=8), 1000),
    ("r8_bs64_exact", dict(n_q_heads=16, n_kv_heads=2, block_size=64, top_k=16), 1024),
]


@pytest.mark.parametrize("name,over,S", DENSE, ids=[c[0] for c in DENSE])
def test_prefill_dense_all_rows(name, over, S):
    """top_k >= nb runs the dense causal kernel: every row against the
    oracle, the selection (every block up to the own one) bit for bit, and
    the output within tolerance of the sparse path (run through the chunked
    entry point, which always takes it)."""
    w = get_workload("tiny_2k", **over)
    assert w.top_k >= -(-S // w.block_size)
    _say(f"[prefill dense] {name} S={S} {w}")
    inp = prefill_inputs(w, seed=31, device="cpu", seq_len=S)
    dinp = {kk: vv.to(DEV) for kk, vv in inp.items()}
    out, sel = _run_prefill(dinp, w.block_size, w.top_k)
    summ, osel, oout = oracle_prefill_rows(inp, w, np.arange(S))
    assert np.array_equal(host_i8(sel).astype(np.int32), osel)
    compare_out(out, oout, name)
    sout, ssel = _chunked(dinp, w.block_size, w.top_k, [0, S], S)
    assert torch.equal(ssel, sel)
    d = (sout.float() - out.float()).abs()
    assert float(d.max()) <= 1e-2 and float(d.mean()) <= 1e-3


def test_prefill_dense_8k_sampled():
    """A short sequence at the 32K workload's heads: 8192 tokens with
    top_k 64 = nb (dense); 128 sampled rows against the oracle."""
    w = get_workload("prefill_32k", top_k=64)
    S = 8192
    _say(f"[prefill dense] S={S} k=64")
    inp = prefill_inputs(w, seed=37, device=DEV, seq_len=S)
    out, sel = _run_prefill(inp, w.block_size, w.top_k)
    rows = sample_rows(S, 128, seed=37)
    summ, osel, oout = oracle_prefill_rows(inp, w, rows)
    rt = torch.as_tensor(rows, device=DEV)
    assert np.array_equal(host_i8(sel[:, :, rt]).astype(np.int32), osel)
    compare_out(out[:, rt], oout, "dense 8K")
    del inp, out, sel
    _free()


# ------------------------------------------------------------------ chunked prefill

def _chunked(inp, bs, k, bounds, C):
    """Run msa_prefill_chunk over the chunks [bounds[i], bounds[i + 1]) of
    a sequence held in caches of capacity C; returns (out, sel) of all rows."""
    B, S, Hq, D = inp["q"].shape
    G = inp["k"].shape[1]
    kc = torch.zeros((B, G, C, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kic = torch.full((B, G, C, inp["k_idx"].shape[3]), 77, dtype=torch.int8, device=DEV)
    bk = torch.zeros((B, G, -(-C // bs), inp["k_idx"].shape[3]), dtype=torch.int8, device=DEV)
    outs, sels = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        # the chunk's keys, values and index keys enter the caches first
        kc[:, :, a:b] = inp["k"][:, :, a:b]
        vc[:, :, a:b] = inp["v"][:, :, a:b]
        kic[:, :, a:b] = inp["k_idx"][:, :, a:b]
        o, sl = msa.msa_prefill_chunk(inp["q"][:, a:b].contiguous(), inp["q_idx"][:, :, a:b].contiguous(), kc, vc,
                                      kic, bk, a, bs, k, return_sel=True)
        outs.append(o)
        sels.append(sl)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1), torch.cat(sels, dim=2)


def test_prefill_query_chunks_batch2():
    """A prefill longer than one query chunk (16384 tokens) with two
    sequences: the chunks slice rows of batch-strided tensors.  Sampled rows
    of both sequences against the oracle, and every row against the same
    sequences prefilled through msa_prefill_chunk in other chunks."""
    w = get_workload("tiny_2k", batch=2, n_q_heads=4, n_kv_heads=2, block_size=64, top_k=6)
    S = 20000
    _say(f"[prefill query chunks] B=2 S={S} {w}")
    inp = prefill_inputs(w, seed=43, device=DEV, seq_len=S)
    out, sel = _run_prefill(inp, w.block_size, w.top_k)
    rows = sample_rows(S, 192, seed=43)
    rt = torch.as_tensor(rows, device=DEV)
    _, osel, oout = oracle_prefill_rows(inp, w, rows)
    assert np.array_equal(host_i8(sel[:, :, rt]).astype(np.int32), osel)
    compare_out(out[:, rt], oout, "query chunks B=2")
    cout, csel = _chunked(inp, w.block_size, w.top_k, [0, 7000, 16384, 16385, S], S)
    assert torch.equal(csel, sel)
    assert torch.equal(cout, out)
    del inp, out, sel, cout, csel
    _free()


CHUNKED = [
    # name, workload overrides, S, chunk bounds, capacity
    ("ragged_gqa4", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=5), 1000, [0, 300, 301, 700, 1000], 1100),
    ("bs128_r8", dict(n_q_heads=16, n_kv_heads=2, block_size=128, top_k=6), 1536, [0, 512, 1024, 1536], 1536),
    ("bs32_k32", dict(n_q_heads=4, n_kv_heads=2, block_size=32, top_k=32), 1500, [0, 40, 1023, 1500], 1600),
    ("batch3", dict(batch=3, n_q_heads=8, n_kv_heads=2, block_size=64, top_k=4), 900, [0, 450, 900], 1000),
]


@pytest.mark.parametrize("name,over,S,bounds,C", CHUNKED, ids=[c[0] for c in CHUNKED])
def test_prefill_chunked_all_rows(name, over, S, bounds, C):
    """A sequence prefilled in chunks against the cache gives, row by row,
    the whole prefill's selection and output (bit for bit), which match the
    oracle."""
    w = get_workload("tiny_2k", **over)
    _say(f"[prefill chunked] {name} S={S} chunks={bounds} C={C}")
    inp = prefill_inputs(w, seed=23, device="cpu", seq_len=S)
    dinp = {kk: vv.to(DEV) for kk, vv in inp.items()}
    cout, csel = _chunked(dinp, w.block_size, w.top_k, bounds, C)
    out, sel = _run_prefill(dinp, w.block_size, w.top_k)
    assert torch.equal(csel, sel), f"{name}: chunked selection differs from the whole prefill"
    assert torch.equal(cout, out), f"{name}: chunked output differs from the whole prefill"
    summ, osel, oout = oracle_prefill_rows(inp, w, np.arange(S))
    assert np.array_equal(host_i8(csel).astype(np.int32), osel)
    compare_out(cout, oout, name)


CHUNKED_VARLEN = [
    # name, workload overrides, sequence lengths, per-sequence counts of each call, capacity
    ("three_seqs_bs64", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=5), [1000, 300, 1],
     [[300, 1, 699], [0, 300, 0], [1, 0, 0]], 1100),
    ("bs128_r8_k6", dict(n_q_heads=16, n_kv_heads=2, block_size=128, top_k=6), [1536, 700],
     [[512, 512, 512], [100, 0, 600]], 1600),
]


@pytest.mark.parametrize("name,over,lens,rounds,C", CHUNKED_VARLEN, ids=[c[0] for c in CHUNKED_VARLEN])
def test_prefill_chunk_varlen_all_rows(name, over, lens, rounds, C):
    """msa_prefill_chunk_varlen: sequences of different lengths, each in its
    own cache, arrive in chunks of different sizes and starts (a sequence may
    add nothing in a call).  Every row of every sequence is bit-equal to
    msa_prefill_chunk on that sequence alone with the same chunks, and
    matches the oracle."""
    w = get_workload("tiny_2k", **over)
    _say(f"[prefill chunk varlen] {name} lengths={lens} counts={rounds} C={C}")
    B, G, bs = len(lens), w.n_kv_heads, w.block_size
    seqs = [prefill_inputs(w, seed=400 + i, device="cpu", seq_len=L) for i, L in enumerate(lens)]
    dseqs = [{kk: vv.to(DEV) for kk, vv in sq.items()} for sq in seqs]
    D, di = seqs[0]["q"].shape[3], seqs[0]["q_idx"].shape[3]
    kc = torch.zeros((B, G, C, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kic = torch.full((B, G, C, di), 77, dtype=torch.int8, device=DEV)
    bk = torch.zeros((B, G, -(-C // bs), di), dtype=torch.int8, device=DEV)
    pos = [0] * B
    outs, sels = [[] for _ in range(B)], [[] for _ in range(B)]
    for r in range(len(rounds[0])):
        starts, counts = list(pos), [rounds[b][r] for b in range(B)]
        for b in range(B):
            a, e = pos[b], pos[b] + counts[b]
            # each sequence's new keys, values and index keys enter its cache first
            kc[b, :, a:e] = dseqs[b]["k"][0, :, a:e]
            vc[b, :, a:e] = dseqs[b]["v"][0, :, a:e]
            kic[b, :, a:e] = dseqs[b]["k_idx"][0, :, a:e]
        q = torch.cat([dseqs[b]["q"][0, pos[b]:pos[b] + counts[b]] for b in range(B)], dim=0).contiguous()
        qi = torch.cat([dseqs[b]["q_idx"][0, :, pos[b]:pos[b] + counts[b]] for b in range(B)], dim=1).contiguous()
        out, sel = msa.msa_prefill_chunk_varlen(q, qi, kc, vc, kic, bk, starts, counts, bs, w.top_k,
                                                return_sel=True)
        o = 0
        for b in range(B):
            n = counts[b]
            outs[b].append(out[o:o + n])
            sels[b].append(sel[:, o:o + n])
            o += n
            pos[b] += n
    torch.cuda.synchronize()
    assert pos == lens
    for b in range(B):
        cout, csel = torch.cat(outs[b], dim=0), torch.cat(sels[b], dim=1)
        bounds = [0]
        for r in range(len(rounds[b])):
            if rounds[b][r] > 0:
                bounds.append(bounds[-1] + rounds[b][r])
        o1, s1 = _chunked(dseqs[b], bs, w.top_k, bounds, C)
        assert torch.equal(csel, s1[0]), f"{name}: sequence {b} selection differs from its own chunked prefill"
        assert torch.equal(cout, o1[0]), f"{name}: sequence {b} output differs from its own chunked prefill"
        _, osel, oout = oracle_prefill_rows(seqs[b], w, np.arange(lens[b]))
        assert np.array_equal(host_i8(csel).astype(np.int32)[None], osel), f"{name}: sequence {b} selection"
        compare_out(cout[None], oout, f"chunk varlen {name} seq {b} (L={lens[b]})")
    del seqs, dseqs, kc, vc, kic, bk
    _free()


def test_prefill_chunked_32k_equals_whole():
    """The 32K workload in four chunks of 8192 queries: bit-identical to the
    whole prefill."""
    w = get_workload("prefill_32k")
    _say("[prefill chunked] 32K in 4 chunks")
    inp = prefill_inputs(w, seed=29, device=DEV)
    out, sel = _run_prefill(inp, w.block_size, w.top_k)
    cout, csel = _chunked(inp, w.block_size, w.top_k, [0, 8192, 16384, 24576, 32768], w.seq_len)
    assert torch.equal(csel, sel)
    assert torch.equal(cout, out)
    del inp, out, sel, cout, csel
    _free()


# ------------------------------------------------------------------ decode

def _decode_case(w, L, B, seed, n_check_units=None):
    _say(f"[decode] L={L} B={B} {w}")
    inp = decode_inputs(w, seed=seed, device=DEV, seq_len=L, batch=B)
    bk = msa.msa_pool_block_keys(inp["k_idx_cache"], w.block_size)
    out, sel = msa.msa_decode(inp["q"], inp["q_idx"], inp["k_cache"], inp["v_cache"], bk, w.block_size,
                              w.top_k, return_sel=True)
    torch.cuda.synchronize()
    summ = O.pool_block_keys(host_i8(inp["k_idx_cache"]), w.block_size)
    assert np.array_equal(host_i8(bk), summ)
    osel, oout = O.decode(host_f32(inp["q"]), host_i8(inp["q_idx"]), HostBf16(inp["k_cache"]),
                          HostBf16(inp["v_cache"]), summ, w.block_size, w.top_k)
    assert np.array_equal(host_i8(sel).astype(np.int32), osel)
    compare_out(out, oout, f"decode L={L}")


@pytest.mark.parametrize("L,B,over", [
    (4096, 2, {}),
    (1000, 3, dict(block_size=64, top_k=5)),
    (100, 1, dict(block_size=128, top_k=4)),
    (5000, 2, dict(n_q_heads=16, n_kv_heads=1, block_size=32, top_k=32)),
    (3000, 2, dict(n_q_heads=8, n_kv_heads=8, top_k=1)),
    # more than 2048 and more than 4096 candidate blocks (8 and 16 per thread)
    (150000, 1, dict(n_q_heads=8, n_kv_heads=1, block_size=64, top_k=16)),
    (300001, 1, dict(n_q_heads=8, n_kv_heads=1, block_size=64, top_k=20)),
    # the largest cache the decode supports: 8193 blocks of 128 (over 1M
    # tokens), 8192 candidates before the own block
    (8193 * 128, 1, dict(n_q_heads=8, n_kv_heads=2, block_size=128, top_k=16)),
])
def test_decode_small(L, B, over):
    w = get_workload("decode_b16_256k", **over)
    _decode_case(w, L, B, seed=L + B)


def test_decode_full_workload():
    w = get_workload("decode_b16_256k")
    _decode_case(w, w.seq_len, w.batch, seed=51)
    _free()


@pytest.mark.parametrize("bs,top_k,L0,steps", [(32, 6, 150, 120), (64, 4, 64, 70)])
def test_decode_generation_steps(bs, top_k, L0, steps):
    """Generation over caches of capacity C: msa_decode_init on L0 cached
    tokens, then one msa_decode_step per new token, crossing block
    boundaries.  Every step's selection and output match the oracle's decode
    over the cache prefix with summaries pooled from all index keys so far;
    the summaries match that pooling after every step, and the appended
    cache rows are the new tokens."""
    w = get_workload("decode_b16_256k", n_q_heads=8, n_kv_heads=2, block_size=bs, top_k=top_k)
    B, C = 2, L0 + steps + 37
    _say(f"[decode generation] bs={bs} k={top_k} L0={L0} steps={steps} C={C}")
    truth = decode_inputs(w, seed=71 + bs, device=DEV, seq_len=C, batch=B)
    tk, tv, tki = truth["k_cache"], truth["v_cache"], truth["k_idx_cache"]
    hk, hv, hki = host_f32(tk), host_f32(tv), host_i8(tki)
    kc, vc = tk.clone(), tv.clone()
    kc[:, :, L0:] = 0
    vc[:, :, L0:] = 0
    kidx = tki.clone()
    kidx[:, :, L0:] = 99  # rows past the cached tokens must not be read
    bk, osum = msa.msa_decode_init(kidx, L0, bs)
    torch.cuda.synchronize()
    nb0 = -(-L0 // bs)
    assert np.array_equal(host_i8(bk)[:, :, :nb0], O.pool_block_keys(hki[:, :, :L0], bs))
    j0 = L0 // bs
    exp_sum = hki[:, :, j0 * bs:L0].astype(np.int64).sum(axis=2)
    assert np.array_equal(host_i8(osum).astype(np.int64), exp_sum)
    for i in range(steps):
        L = L0 + i + 1
        pos = L - 1
        qs = decode_inputs(w, seed=5000 + i, device=DEV, seq_len=1, batch=B)
        out, sel = msa.msa_decode_step(qs["q"], qs["q_idx"], tk[:, :, pos].contiguous(), tv[:, :, pos].contiguous(),
                                       tki[:, :, pos].contiguous(), kc, vc, osum, bk, L, bs, top_k,
                                       return_sel=True)
        torch.cuda.synchronize()
        summ = O.pool_block_keys(hki[:, :, :L], bs)
        assert np.array_equal(host_i8(bk)[:, :, :-(-L // bs)], summ), f"summaries after step L={L}"
        osel, oout = O.decode(host_f32(qs["q"]), host_i8(qs["q_idx"]), hk[:, :, :L], hv[:, :, :L], summ, bs,
                              top_k)
        assert np.array_equal(host_i8(sel).astype(np.int32), osel), f"selection at L={L}"
        compare_out(out, oout, f"decode step L={L}")
    Lend = L0 + steps
    assert torch.equal(kc[:, :, :Lend], tk[:, :, :Lend]) and torch.equal(vc[:, :, :Lend], tv[:, :, :Lend])
    assert int(kc[:, :, Lend:].abs().sum()) == 0


def test_decode_varlen_rows():
    """msa_decode_varlen over a ragged batch (1 to 70000 cached tokens in
    caches of 70001, partial and full last blocks): each sequence's
    selection and output bit-equal to msa_decode on that sequence alone and
    matching the oracle; msa_decode_init_varlen's summaries and open-block
    sums equal the pooling of each sequence's own tokens (rows past them are
    never read)."""
    w = get_workload("decode_b16_256k", n_q_heads=8, n_kv_heads=2, block_size=64, top_k=8)
    lens = [1, 100, 128, 4097, 70000]
    B, C, bs, k = len(lens), max(lens) + 1, w.block_size, w.top_k
    _say(f"[decode varlen] lengths={lens} C={C} {w}")
    inp = decode_inputs(w, seed=91, device=DEV, seq_len=C, batch=B)
    kidx = inp["k_idx_cache"].clone()
    for b, L in enumerate(lens):
        kidx[b, :, L:] = 99
    bk, osum = msa.msa_decode_init_varlen(kidx, lens, bs)
    out, sel = msa.msa_decode_varlen(inp["q"], inp["q_idx"], inp["k_cache"], inp["v_cache"], bk, lens, bs, k,
                                     return_sel=True)
    torch.cuda.synchronize()
    hki = host_i8(inp["k_idx_cache"])
    for b, L in enumerate(lens):
        nb = -(-L // bs)
        summ = O.pool_block_keys(hki[b:b + 1, :, :L], bs)
        assert np.array_equal(host_i8(bk)[b:b + 1, :, :nb], summ), f"summaries of sequence {b}"
        j0 = L // bs
        assert np.array_equal(host_i8(osum)[b].astype(np.int64),
                              hki[b, :, j0 * bs:L].astype(np.int64).sum(axis=1)), f"open sums of sequence {b}"
        o1, s1 = msa.msa_decode(inp["q"][b:b + 1].contiguous(), inp["q_idx"][b:b + 1].contiguous(),
                                inp["k_cache"][b:b + 1, :, :L].contiguous(), inp["v_cache"][b:b + 1, :, :L].contiguous(),
                                bk[b:b + 1, :, :nb].contiguous(), bs, k, return_sel=True)
        torch.cuda.synchronize()
        assert torch.equal(sel[b:b + 1], s1), f"sequence {b}: selection differs from msa_decode alone"
        assert torch.equal(out[b:b + 1], o1), f"sequence {b}: output differs from msa_decode alone"
        osel, oout = O.decode(host_f32(inp["q"][b:b + 1]), host_i8(inp["q_idx"][b:b + 1]),
                              HostBf16(inp["k_cache"][b:b + 1, :, :L]), HostBf16(inp["v_cache"][b:b + 1, :, :L]),
                              summ, bs, k)
        assert np.array_equal(host_i8(sel[b:b + 1]).astype(np.int32), osel), f"selection of sequence {b}"
        compare_out(out[b:b + 1], oout, f"decode varlen L={L}")
    del inp, kidx, bk, osum, out, sel
    _free()


def test_decode_varlen_device_lengths():
    """Lengths in device memory, read by the kernels: bit-equal to the
    host-lengths call for lengths in range; a length outside 1 .. C (0,
    C + 1, -7) gives a zero output row and sel -1, leaves the other
    sequences' rows unchanged, and an out-of-range step appends nothing."""
    w = get_workload("decode_b16_256k", n_q_heads=8, n_kv_heads=2, block_size=64, top_k=8)
    C, bs, k = 9000, w.block_size, w.top_k
    good = [1, 900, 65, 9000, 4000, 3000]
    bad = [1, 0, 65, C + 1, -7, 3000]
    B = len(good)
    _say(f"[decode varlen device] lengths={good} / {bad} C={C}")
    inp = decode_inputs(w, seed=93, device=DEV, seq_len=C, batch=B)
    bk, osum = msa.msa_decode_init_varlen(inp["k_idx_cache"], good, bs)
    args = (inp["q"], inp["q_idx"], inp["k_cache"], inp["v_cache"], bk)
    oh, sh = msa.msa_decode_varlen(*args, good, bs, k, return_sel=True)
    od, sd = msa.msa_decode_varlen(*args, torch.tensor(good, dtype=torch.int32, device=DEV), bs, k, return_sel=True)
    ob, sb = msa.msa_decode_varlen(*args, torch.tensor(bad, dtype=torch.int32, device=DEV), bs, k, return_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(od, oh) and torch.equal(sd, sh), "device lengths differ from host lengths"
    for b in range(B):
        if 1 <= bad[b] <= C:
            assert torch.equal(ob[b], oh[b]) and torch.equal(sb[b], sh[b]), f"sequence {b} changed"
        else:
            assert int(ob[b].float().abs().sum()) == 0 and bool((sb[b] == -1).all()), f"sequence {b} not empty"
    # a step with out-of-range lengths leaves those sequences' state alone
    kc, vc, bk2, os2 = inp["k_cache"].clone(), inp["v_cache"].clone(), bk.clone(), osum.clone()
    new = decode_inputs(w, seed=94, device=DEV, seq_len=1, batch=B)
    lens_next = torch.tensor([x + 1 if 1 <= x < C else x for x in bad], dtype=torch.int32, device=DEV)
    o, s_ = msa.msa_decode_step_varlen(new["q"], new["q_idx"], new["k_cache"][:, :, 0].contiguous(),
                                       new["v_cache"][:, :, 0].contiguous(), new["k_idx_cache"][:, :, 0].contiguous(),
                                       kc, vc, os2, bk2, lens_next, bs, k, return_sel=True)
    torch.cuda.synchronize()
    for b in range(B):
        if not 1 <= bad[b] <= C:
            assert torch.equal(kc[b], inp["k_cache"][b]) and torch.equal(vc[b], inp["v_cache"][b])
            assert torch.equal(bk2[b], bk[b]) and torch.equal(os2[b], osum[b])
            assert int(o[b].float().abs().sum()) == 0 and bool((s_[b] == -1).all())
    del inp, kc, vc
    _free()


def test_decode_step_varlen_generation():
    """Ragged generation: msa_decode_init_varlen on 1, 63, 64 and 200 cached
    tokens, then 70 msa_decode_step_varlen steps, each sequence appending at
    its own position (every one crosses a block boundary).  Every step's
    selection and output match the oracle's decode of each sequence's prefix
    with summaries pooled from its index keys so far, the summaries match
    that pooling after every step, and the caches end as the new tokens."""
    w = get_workload("decode_b16_256k", n_q_heads=8, n_kv_heads=2, block_size=64, top_k=4)
    L0s, steps, bs, k = [1, 63, 64, 200], 70, 64, 4
    B, C = len(L0s), max(L0s) + steps + 5
    _say(f"[decode generation varlen] L0={L0s} steps={steps} C={C}")
    truth = decode_inputs(w, seed=171, device=DEV, seq_len=C, batch=B)
    tk, tv, tki = truth["k_cache"], truth["v_cache"], truth["k_idx_cache"]
    hk, hv, hki = host_f32(tk), host_f32(tv), host_i8(tki)
    kc, vc, kidx = tk.clone(), tv.clone(), tki.clone()
    for b, L0 in enumerate(L0s):
        kc[b, :, L0:] = 0
        vc[b, :, L0:] = 0
        kidx[b, :, L0:] = 99
    bk, osum = msa.msa_decode_init_varlen(kidx, L0s, bs)
    for i in range(steps):
        lens = [L0 + i + 1 for L0 in L0s]
        pos = torch.tensor([L - 1 for L in lens], device=DEV)
        ar = torch.arange(B, device=DEV)
        qs = decode_inputs(w, seed=7000 + i, device=DEV, seq_len=1, batch=B)
        k_new = tk[ar, :, pos].contiguous()
        v_new = tv[ar, :, pos].contiguous()
        ki_new = tki[ar, :, pos].contiguous()
        out, sel = msa.msa_decode_step_varlen(qs["q"], qs["q_idx"], k_new, v_new, ki_new, kc, vc, osum, bk, lens,
                                              bs, k, return_sel=True)
        torch.cuda.synchronize()
        for b, L in enumerate(lens):
            summ = O.pool_block_keys(hki[b:b + 1, :, :L], bs)
            assert np.array_equal(host_i8(bk)[b:b + 1, :, :-(-L // bs)], summ), f"summaries of {b} at L={L}"
            osel, oout = O.decode(host_f32(qs["q"][b:b + 1]), host_i8(qs["q_idx"][b:b + 1]), hk[b:b + 1, :, :L],
                                  hv[b:b + 1, :, :L], summ, bs, k)
            assert np.array_equal(host_i8(sel[b:b + 1]).astype(np.int32), osel), f"selection of {b} at L={L}"
            compare_out(out[b:b + 1], oout, f"decode step varlen seq {b} L={L}")
    for b, L0 in enumerate(L0s):
        Lend = L0 + steps
        assert torch.equal(kc[b, :, :Lend], tk[b, :, :Lend]) and torch.equal(vc[b, :, :Lend], tv[b, :, :Lend])
        assert int(kc[b, :, Lend:].abs().sum()) == 0


def test_decode_matches_last_prefill_row():
    w = get_workload("prefill_32k")
    S = 5000
    _say(f"[decode vs prefill] S={S}")
    inp = prefill_inputs(w, seed=61, device=DEV, seq_len=S)
    out, sel = _run_prefill(inp, w.block_size, w.top_k)
    bk = msa.msa_pool_block_keys(inp["k_idx"], w.block_size)
    dout, dsel = msa.msa_decode(inp["q"][:, S - 1].contiguous(), inp["q_idx"][:, :, S - 1].contiguous(),
                                inp["k"], inp["v"], bk, w.block_size, w.top_k, return_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(dsel, sel[:, :, S - 1])
    d = (dout.float() - out[:, S - 1].float()).abs()
    assert float(d.max()) <= 1e-2


# ------------------------------------------------------------------ ragged batch and the short-sequence switch

VARLEN = [
    # name, workload overrides, sequence lengths (one longer than a 16384-token query chunk, a 1-token
    # sequence, an empty one, lengths that are not multiples of the block size)
    ("mixed_bs64_k6", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=6), [1, 300, 20000, 129, 4096, 0, 64]),
    ("bs128_r8_k16", dict(n_q_heads=16, n_kv_heads=2, block_size=128, top_k=16), [3000, 777, 5000, 1]),
]


@pytest.mark.parametrize("name,over,lens", VARLEN, ids=[c[0] for c in VARLEN])
def test_prefill_varlen_all_rows(name, over, lens):
    """msa_prefill_varlen over sequences packed along the token axis: every
    row of every sequence against the oracle of that sequence alone, and bit
    for bit the rows msa_prefill gives each sequence on its own."""
    w = get_workload("tiny_2k", **over)
    _say(f"[prefill varlen] {name} lengths={lens}")
    seqs = [prefill_inputs(w, seed=300 + i, device=DEV, seq_len=L) if L > 0 else None for i, L in enumerate(lens)]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    live = [s for s in seqs if s is not None]
    q = torch.cat([s["q"][0] for s in live], dim=0).contiguous()
    k = torch.cat([s["k"][0] for s in live], dim=1).contiguous()
    v = torch.cat([s["v"][0] for s in live], dim=1).contiguous()
    qi = torch.cat([s["q_idx"][0] for s in live], dim=1).contiguous()
    ki = torch.cat([s["k_idx"][0] for s in live], dim=1).contiguous()
    out, sel = msa.msa_prefill_varlen(q, k, v, qi, ki, cu, w.block_size, w.top_k, return_sel=True)
    torch.cuda.synchronize()
    for i, s in enumerate(seqs):
        if s is None:
            continue
        a, b = cu[i], cu[i + 1]
        o1, s1 = _run_prefill(s, w.block_size, w.top_k)
        assert torch.equal(out[a:b], o1[0]), f"{name}: sequence {i} output differs from its own msa_prefill"
        assert torch.equal(sel[:, a:b], s1[0]), f"{name}: sequence {i} selection differs from its own msa_prefill"
        rows = np.arange(b - a)
        _, osel, oout, st = oracle_prefill_rows_pooled(s, w, rows)
        assert np.array_equal(host_i8(sel[:, a:b]).astype(np.int32)[None], osel), f"{name}: sequence {i} selection"
        compare_rounded(out[a:b][None], oout, f"varlen {name} seq {i} (L={b - a})")
    del seqs, live, q, k, v, qi, ki, out, sel
    _free()


def test_prefill_switched_short_is_standard_attention():
    """Below the threshold msa_prefill_switched computes standard causal GQA
    attention (every earlier key, whatever top_k), which the oracle gives with
    a selection that keeps every block; sel is all -1.  At or above it, the
    call is msa_prefill, bit for bit."""
    w = get_workload("tiny_2k", n_q_heads=16, n_kv_heads=2, block_size=64, top_k=4)
    S = 3000  # 47 blocks: top_k 4 would select; the switch does not
    _say(f"[prefill switched] S={S} {w}")
    inp = prefill_inputs(w, seed=55, device=DEV, seq_len=S)
    sel = torch.zeros((1, w.n_kv_heads, S, w.top_k), dtype=torch.int32, device=DEV)
    out, dense = msa.msa_prefill_switched(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], w.block_size,
                                          w.top_k, sel=sel)
    torch.cuda.synchronize()
    assert dense
    assert bool((sel == -1).all())
    nb = -(-S // w.block_size)
    rows = np.arange(S)
    _, osel, oout, st = oracle_prefill_rows_pooled(inp, w, rows, top_k=nb)
    compare_rounded(out, oout, "switched: standard attention, 3000 tokens")
    # the same data through MSA differs: top_k 4 keeps 4 of up to 47 blocks
    msa_out, _ = _run_prefill(inp, w.block_size, w.top_k)
    assert float((msa_out.float() - out.float()).abs().max()) > 0.05
    # at or above the threshold: msa_prefill exactly
    out2, dense2 = msa.msa_prefill_switched(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], w.block_size,
                                            w.top_k, dense_below=2000)
    torch.cuda.synchronize()
    assert not dense2
    assert torch.equal(out2, msa_out)
    del inp, out, out2, msa_out, sel
    _free()
