"""GPU parity of the training path: msa_prefill_lse (forward + log-sum-exp)
and msa_prefill_backward (dq, dk, dv with the selection fixed) against the
CPU oracle.

The log-sum-exp is fp32 arithmetic on bf16 inputs: within 1e-3 of the
oracle's fp64 value.  A gradient element is a bf16-rounded sum whose terms
each pass through bf16 rounding (relative error <= 2^-9) two or three more
times than the forward's do: P or dS as an MFMA operand, the per-block dq
partial, and delta taken from the bf16 output: at most about 3 * 2^-9 of
the terms' magnitude.  dq and dk are sums of terms that cancel (the dS of a
query row sum to zero), so relative to the result the error can be a small
multiple of that; the comparison allows a factor of about two, relative to
the gradient's own scale (floored at 1e-2, for gradients that are exactly
zero, e.g. with a single attended key), per tensor:
  max |gpu - bf16(oracle)|  <= 2e-2 * max |oracle|
  mean |gpu - bf16(oracle)| <= 1e-2 * mean |oracle|.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_33_amd as msa
from oracle import msa_oracle as O
from synth import get_workload, grad_output, prefill_inputs, sample_rows
from tests.helpers import host_f32, host_i8, oracle_kv_grads_pooled, oracle_query_grads_pooled, record

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LSE_ABS = 1e-3
GRAD_MAX_REL = 2e-2
GRAD_MEAN_REL = 1e-2
GRAD_FLOOR = 1e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def compare_grad(gpu_bf16, oracle_f64, what):
    g = host_f32(gpu_bf16).astype(np.float64)
    ref = O.round_to_bf16(oracle_f64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU gradient"
    d = np.abs(g - ref)
    # the gradient's own scale, floored at 1e-2: a gradient that is zero in
    # exact arithmetic (one attended key gives dS = 0) is held to an
    # absolute bar instead
    scale_max = max(float(np.abs(ref).max()), GRAD_FLOOR)
    scale_mean = max(float(np.abs(ref).mean()), GRAD_FLOOR)
    max_rel, mean_rel = float(d.max()) / scale_max, float(d.mean()) / scale_mean
    _say(f"  {what}: max_rel={max_rel:.2e} mean_rel={mean_rel:.2e} (max|ref|={scale_max:.3g})")
    record(what, {"elements": int(d.size), "grad_max_rel": max_rel, "grad_mean_rel": mean_rel,
                  "max_abs_oracle": float(np.abs(ref).max()), "mean_abs_oracle": float(np.abs(ref).mean()),
                  "bars": [GRAD_MAX_REL, GRAD_MEAN_REL]})
    assert max_rel <= GRAD_MAX_REL and mean_rel <= GRAD_MEAN_REL, (
        f"{what}: max|err|/max|ref| = {max_rel:.3e} (<= {GRAD_MAX_REL}), mean|err|/mean|ref| = {mean_rel:.3e} "
        f"(<= {GRAD_MEAN_REL}), worst at {np.unravel_index(int(d.argmax()), d.shape)}")


def _block_pairs(nb, G, fixed, n_random, seed):
    """(block, group) pairs: the fixed ones, then n_random distinct seeded
    ones not among them."""
    rng = np.random.default_rng(seed)
    pairs = [tuple(p) for p in fixed]
    while len(pairs) < len(fixed) + n_random:
        p = (int(rng.integers(nb)), int(rng.integers(G)))
        if p not in pairs:
            pairs.append(p)
    return pairs


def _gather_blocks(x, pairs, bs):
    """Rows of key block j in group g of x [B, G, S, D], stacked per pair:
    [B, len(pairs), bs, D]."""
    return torch.stack([x[:, g, j * bs:(j + 1) * bs] for j, g in pairs], dim=1)


def _forward_backward(inp, dout, bs, top_k):
    out, sel, lse = msa.msa_prefill_lse(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], bs, top_k)
    dq, dk, dv = msa.msa_prefill_backward(inp["q"], inp["k"], inp["v"], out, dout, lse, sel, bs)
    torch.cuda.synchronize()
    return out, sel, lse, dq, dk, dv


# ------------------------------------------------------------------ small cases, every element

SMALL = [
    # name, workload overrides, seq_len
    ("tiny_2k", {}, None),
    ("ragged_gqa4_bs64", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=5), 1000),
    ("batch2_r1_bs32", dict(batch=2, n_q_heads=2, n_kv_heads=2, block_size=32, top_k=4), 600),
    ("r16_bs128", dict(n_q_heads=16, n_kv_heads=1, block_size=128, top_k=3), 777),
    ("topk1_own_only", dict(n_q_heads=8, n_kv_heads=1, top_k=1), 700),
    ("dense_sel_bs64", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=32), 1100),
    ("single_block", dict(n_q_heads=8, n_kv_heads=1, block_size=128, top_k=4), 100),
    ("r2_bs64_k2", dict(n_q_heads=4, n_kv_heads=2, block_size=64, top_k=2), 513),
    ("one_token", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=4), 1),
    ("three_tokens_b3_r1", dict(batch=3, n_q_heads=2, n_kv_heads=2, block_size=32, top_k=2), 3),
]


@pytest.mark.parametrize("name,over,S", SMALL, ids=[c[0] for c in SMALL])
def test_prefill_lse_small(name, over, S):
    w = get_workload("tiny_2k", **over)
    _say(f"[lse small] {name} S={S or w.seq_len}")
    inp = prefill_inputs(w, seed=5, device="cpu", seq_len=S)
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    out, sel, lse = msa.msa_prefill_lse(dinp["q"], dinp["k"], dinp["v"], dinp["q_idx"], dinp["k_idx"],
                                        w.block_size, w.top_k)
    ref_out = msa.msa_prefill(dinp["q"], dinp["k"], dinp["v"], dinp["q_idx"], dinp["k_idx"], w.block_size, w.top_k)
    torch.cuda.synchronize()
    # the log-sum-exp output changes nothing else
    assert torch.equal(out, ref_out), f"{name}: msa_prefill_lse output differs from msa_prefill"
    Sn = inp["q"].shape[1]
    rows = np.arange(Sn)
    summ = O.pool_block_keys(inp["k_idx"].numpy(), w.block_size)
    osel = O.select_blocks(inp["q_idx"].numpy(), summ, w.block_size, w.top_k, rows)
    assert np.array_equal(host_i8(sel).astype(np.int32), osel), f"{name}: selection differs"
    olse = O.lse_rows(host_f32(inp["q"]), host_f32(inp["k"]), host_f32(inp["v"]), osel, rows, w.block_size)
    err = np.abs(lse.cpu().numpy().astype(np.float64) - olse)
    assert float(err.max()) <= LSE_ABS, f"{name}: lse max_abs={err.max():.3e}"


def test_backward_custom_scale():
    """A softmax scale other than 1/sqrt(D), passed to both calls."""
    w = get_workload("tiny_2k", n_q_heads=8, n_kv_heads=2, block_size=64, top_k=4)
    S, scale = 900, 0.05
    _say(f"[backward scale] S={S} scale={scale}")
    inp = prefill_inputs(w, seed=13, device="cpu", seq_len=S)
    dout = grad_output(w, seed=13, device="cpu", seq_len=S)
    d = {k: v.to(DEV) for k, v in inp.items()}
    out, sel, lse = msa.msa_prefill_lse(d["q"], d["k"], d["v"], d["q_idx"], d["k_idx"], w.block_size, w.top_k,
                                        softmax_scale=scale)
    dq, dk, dv = msa.msa_prefill_backward(d["q"], d["k"], d["v"], out, dout.to(DEV), lse, sel, w.block_size,
                                          softmax_scale=scale)
    torch.cuda.synchronize()
    summ = O.pool_block_keys(inp["k_idx"].numpy(), w.block_size)
    osel = O.select_blocks(inp["q_idx"].numpy(), summ, w.block_size, w.top_k)
    assert np.array_equal(host_i8(sel).astype(np.int32), osel)
    hq, hk, hv = host_f32(inp["q"]), host_f32(inp["k"]), host_f32(inp["v"])
    olse = O.lse_rows(hq, hk, hv, osel, np.arange(S), w.block_size, scale=scale)
    assert float(np.abs(lse.cpu().numpy() - olse).max()) <= LSE_ABS
    rq, rk, rv = O.backward(hq, hk, hv, host_f32(dout), osel, w.block_size, scale=scale)
    compare_grad(dq, rq, "scale dq")
    compare_grad(dk, rk, "scale dk")
    compare_grad(dv, rv, "scale dv")


@pytest.mark.parametrize("name,over,S", SMALL, ids=[c[0] for c in SMALL])
def test_backward_small_all_elements(name, over, S):
    w = get_workload("tiny_2k", **over)
    _say(f"[backward small] {name} S={S or w.seq_len}")
    inp = prefill_inputs(w, seed=9, device="cpu", seq_len=S)
    dout = grad_output(w, seed=9, device="cpu", seq_len=S)
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    _, sel, _, dq, dk, dv = _forward_backward(dinp, dout.to(DEV), w.block_size, w.top_k)
    Sn = inp["q"].shape[1]
    summ = O.pool_block_keys(inp["k_idx"].numpy(), w.block_size)
    osel = O.select_blocks(inp["q_idx"].numpy(), summ, w.block_size, w.top_k)
    assert np.array_equal(host_i8(sel).astype(np.int32), osel), f"{name}: selection differs"
    rq, rk, rv = O.backward(host_f32(inp["q"]), host_f32(inp["k"]), host_f32(inp["v"]), host_f32(dout), osel,
                            w.block_size)
    assert rq.shape == (w.batch, Sn, w.n_q_heads, 128)
    compare_grad(dq, rq, f"{name} dq")
    compare_grad(dk, rk, f"{name} dk")
    compare_grad(dv, rv, f"{name} dv")


# ------------------------------------------------------------------ full size

def test_backward_32k_sampled_and_sums():
    """Prefill 32K (64 query heads, 8 groups, block 128, top_k 16): dq on
    every row and dk, dv of 48 (block, group) pairs against the oracle; over every
    key, the closed-form sums (dv rows of a group sum to its heads' dout
    rows, dk rows sum to 0)."""
    w = get_workload("prefill_32k")
    S, bs = w.seq_len, w.block_size
    _say(f"[backward full] prefill_32k S={S}")
    inp = prefill_inputs(w, seed=33, device=DEV)
    dout = grad_output(w, seed=33, device=DEV)
    _, sel, _, dq, dk, dv = _forward_backward(inp, dout, bs, w.top_k)
    gsel = host_i8(sel).astype(np.int32)
    del sel
    _free()
    # sums over every key of each group (fp64 on the host)
    gdv = host_f32(dv).astype(np.float64)
    gdk = host_f32(dk).astype(np.float64)
    dsum = host_f32(dout).astype(np.float64).reshape(w.batch, S, w.n_kv_heads, -1, 128).sum(axis=(1, 3))
    np.testing.assert_allclose(gdv.sum(axis=2), dsum, rtol=0, atol=2e-3 * np.abs(gdv).sum(axis=2).max())
    assert np.abs(gdk.sum(axis=2)).max() <= 2e-3 * np.abs(gdk).sum(axis=2).max()
    # oracle on samples, with its own selection of every row
    _say("[backward full] oracle selection of every row")
    summ = O.pool_block_keys(host_i8(inp["k_idx"]), bs)
    osel = O.select_blocks(host_i8(inp["q_idx"]), summ, bs, w.top_k)
    assert np.array_equal(gsel, osel), "selection differs"
    rows = np.arange(S)
    _say(f"[backward full] oracle dq on every row ({S}, worker processes)")
    rq, st = oracle_query_grads_pooled(inp, dout, osel, rows, bs)
    _say(f"[backward full] oracle dq: {st}")
    compare_grad(dq, rq, "32k dq (every row)")
    del rq
    # dk, dv of 48 (block, group) pairs: block 0 (kept by the most queries),
    # an early block (~6000 queries of its group), a middle one, the last
    # one, and 44 seeded ones
    pairs = _block_pairs(S // bs, w.n_kv_heads, [(0, 2), (5, 3), (140, 6), (255, 0)], 44, seed=33)
    _say(f"[backward full] oracle dk, dv of {len(pairs)} (block, group) pairs (worker processes)")
    rk, rv, st = oracle_kv_grads_pooled(inp, dout, osel, pairs, bs)
    _say(f"[backward full] oracle dk, dv: {st}")
    compare_grad(_gather_blocks(dk, pairs, bs), rk, f"32k dk ({len(pairs)} blocks)")
    compare_grad(_gather_blocks(dv, pairs, bs), rv, f"32k dv ({len(pairs)} blocks)")
    del inp, dout, dq, dk, dv
    _free()


def test_backward_structured_128k_sampled_and_sums():
    """The structured 128K workload (hot blocks kept by most queries of their
    group, so some CSR rows are very long): dq on 4096 sampled rows and dk, dv
    of the last block and 8 seeded (block, group) pairs against the oracle; the closed-form sums over every key."""
    w = get_workload("structured_128k")
    S, bs = w.seq_len, w.block_size
    _say(f"[backward full] structured_128k S={S}")
    inp = prefill_inputs(w, seed=41, device=DEV)
    dout = grad_output(w, seed=41, device=DEV)
    _, sel, _, dq, dk, dv = _forward_backward(inp, dout, bs, w.top_k)
    gsel = host_i8(sel).astype(np.int32)
    del sel
    _free()
    gdv = host_f32(dv).astype(np.float64)
    gdk = host_f32(dk).astype(np.float64)
    dsum = host_f32(dout).astype(np.float64).reshape(w.batch, S, w.n_kv_heads, -1, 128).sum(axis=(1, 3))
    np.testing.assert_allclose(gdv.sum(axis=2), dsum, rtol=0, atol=2e-3 * np.abs(gdv).sum(axis=2).max())
    assert np.abs(gdk.sum(axis=2)).max() <= 2e-3 * np.abs(gdk).sum(axis=2).max()
    del gdv, gdk
    _say("[backward full] oracle selection of every row")
    summ = O.pool_block_keys(host_i8(inp["k_idx"]), bs)
    osel = O.select_blocks(host_i8(inp["q_idx"]), summ, bs, w.top_k)
    assert np.array_equal(gsel, osel), "selection differs"
    rows = sample_rows(S, 4096, 41)
    _say(f"[backward full] oracle dq on {len(rows)} rows (worker processes)")
    rq, st = oracle_query_grads_pooled(inp, dout, osel[:, :, rows], rows, bs)
    _say(f"[backward full] oracle dq: {st}")
    compare_grad(dq[:, torch.as_tensor(rows, device=DEV)], rq, "128k dq (sampled rows)")
    pairs = _block_pairs(S // bs, w.n_kv_heads, [(S // bs - 1, 5)], 8, seed=41)
    _say(f"[backward full] oracle dk, dv of {len(pairs)} (block, group) pairs (worker processes)")
    rk, rv, st = oracle_kv_grads_pooled(inp, dout, osel, pairs, bs)
    _say(f"[backward full] oracle dk, dv: {st}")
    compare_grad(_gather_blocks(dk, pairs, bs), rk, f"128k dk ({len(pairs)} blocks)")
    compare_grad(_gather_blocks(dv, pairs, bs), rv, f"128k dv ({len(pairs)} blocks)")
    del inp, dout, dq, dk, dv
    _free()


# ------------------------------------------------------------------ query passes (bounded workspace)

def _pass_workspace(w, S, frac):
    """A workspace between the least one (passes of 256 query rows) and the
    full one: frac 0 gives the least, 1 the full size."""
    dims = msa.make_dims(w.batch, S, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k, head_dim=128)
    lo, hi = msa.msa_workspace_bytes(msa.MSA_OP_BACKWARD, dims)
    size = lo + int((hi - lo) * frac)
    return torch.empty(size, dtype=torch.uint8, device=DEV), lo, hi


def _close_to_one_pass(a, b, what):
    """dk or dv from passes against the one-pass result: both round fp32 sums
    of the same terms, added in another order, to bf16."""
    x, y = a.float(), b.float()
    d = (x - y).abs()
    scale_max = max(float(y.abs().max()), GRAD_FLOOR)
    scale_mean = max(float(y.abs().mean()), GRAD_FLOOR)
    max_rel, mean_rel = float(d.max()) / scale_max, float(d.mean()) / scale_mean
    _say(f"  {what} vs one pass: max_rel={max_rel:.2e} mean_rel={mean_rel:.2e}")
    assert max_rel <= 2.0 ** -7 and mean_rel <= 2.0 ** -8, (what, max_rel, mean_rel)


PASS_CASES = [
    # name, workload overrides, seq_len, place of the workspace between least and full
    ("tiny_2k_least", {}, None, 0.0),
    ("tiny_2k_middle", {}, None, 0.4),
    # (with one head per group and few kept blocks the fp32 sums outweigh the
    # saved partials: the least workspace is then the full one)
    ("batch2_r2_bs32_least", dict(batch=2, n_q_heads=4, n_kv_heads=2, block_size=32, top_k=8), 600, 0.0),
    ("ragged_gqa4_bs64_least", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=5), 1000, 0.0),
    ("r16_bs128_least", dict(n_q_heads=16, n_kv_heads=1, block_size=128, top_k=3), 777, 0.0),
    ("dense_sel_bs64_least", dict(n_q_heads=8, n_kv_heads=2, block_size=64, top_k=32), 1100, 0.0),
]


@pytest.mark.parametrize("name,over,S", [c[:3] for c in PASS_CASES], ids=[c[0] for c in PASS_CASES])
def test_backward_passes_small(name, over, S):
    """A workspace smaller than the full one runs the query rows in passes:
    dq equals the one-pass result bit for bit (each query's partials do not
    depend on which rows share its pass), dk and dv agree with the one-pass
    result to bf16 rounding and with the oracle to the gradient bar."""
    frac = {c[0]: c[3] for c in PASS_CASES}[name]
    w = get_workload("tiny_2k", **over)
    Sn = S or w.seq_len
    inp = prefill_inputs(w, seed=17, device="cpu", seq_len=S)
    dout = grad_output(w, seed=17, device="cpu", seq_len=S)
    d = {k: v.to(DEV) for k, v in inp.items()}
    ws, lo, hi = _pass_workspace(w, Sn, frac)
    _say(f"[backward passes] {name} S={Sn} workspace={ws.numel()} (least {lo}, full {hi})")
    assert lo < hi
    out, sel, lse, dq1, dk1, dv1 = _forward_backward(d, dout.to(DEV), w.block_size, w.top_k)
    dq, dk, dv = msa.msa_prefill_backward(d["q"], d["k"], d["v"], out, dout.to(DEV), lse, sel, w.block_size,
                                          workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq1), f"{name}: dq from passes differs from one pass"
    _close_to_one_pass(dk, dk1, f"{name} dk")
    _close_to_one_pass(dv, dv1, f"{name} dv")
    summ = O.pool_block_keys(inp["k_idx"].numpy(), w.block_size)
    osel = O.select_blocks(inp["q_idx"].numpy(), summ, w.block_size, w.top_k)
    assert np.array_equal(host_i8(sel).astype(np.int32), osel), f"{name}: selection differs"
    rq, rk, rv = O.backward(host_f32(inp["q"]), host_f32(inp["k"]), host_f32(inp["v"]), host_f32(dout), osel,
                            w.block_size)
    compare_grad(dq, rq, f"{name} dq")
    compare_grad(dk, rk, f"{name} dk")
    compare_grad(dv, rv, f"{name} dv")


def test_backward_passes_32k():
    """Prefill 32K with a workspace of about an eighth of the full one
    (passes of a few thousand query rows): dq equals the one-pass result,
    dk and dv agree with it to bf16 rounding."""
    w = get_workload("prefill_32k")
    S, bs = w.seq_len, w.block_size
    inp = prefill_inputs(w, seed=35, device=DEV)
    dout = grad_output(w, seed=35, device=DEV)
    out, sel, lse, dq1, dk1, dv1 = _forward_backward(inp, dout, bs, w.top_k)
    ws, lo, hi = _pass_workspace(w, S, 0.125)
    _say(f"[backward passes] prefill_32k workspace={ws.numel()} (least {lo}, full {hi})")
    dq, dk, dv = msa.msa_prefill_backward(inp["q"], inp["k"], inp["v"], out, dout, lse, sel, bs, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq1), "32k: dq from passes differs from one pass"
    _close_to_one_pass(dk, dk1, "32k dk")
    _close_to_one_pass(dv, dv1, "32k dv")
    del inp, dout, out, sel, lse, dq1, dk1, dv1, ws, dq, dk, dv
    _free()


def _check_long_backward(w, inp, dout, sel, dq, dk, dv, seed, g, n_rows=128):
    """Checks of a long backward: the closed-form sums over every key (fp64
    on the GPU), dq of sampled rows and dk, dv of the last block of group g
    against the oracle."""
    from tests.helpers import HostBf16
    S, bs, K = w.seq_len, w.block_size, w.top_k
    B, G, r = w.batch, w.n_kv_heads, w.n_q_heads // w.n_kv_heads
    # closed-form sums over every key (fp64 on the GPU, in slices of rows)
    step = 1 << 16
    sv = torch.zeros(B, G, 128, dtype=torch.float64, device=DEV)
    sk = torch.zeros_like(sv)
    av = torch.zeros_like(sv)
    ak = torch.zeros_like(sv)
    sd = torch.zeros_like(sv)
    for s0 in range(0, S, step):
        x = dv[:, :, s0:s0 + step].double()
        sv += x.sum(2)
        av += x.abs().sum(2)
        x = dk[:, :, s0:s0 + step].double()
        sk += x.sum(2)
        ak += x.abs().sum(2)
        n = min(step, S - s0)
        sd += dout[:, s0:s0 + step].double().view(B, n, G, r, 128).sum((1, 3))
    assert float((sv - sd).abs().max()) <= 2e-3 * float(av.max()), "dv rows do not sum to the dout rows"
    assert float(sk.abs().max()) <= 2e-3 * float(ak.max()), "dk rows do not sum to zero"
    # oracle: selection and dq of sampled rows
    summ = O.pool_block_keys(host_i8(inp["k_idx"]), bs)
    qi = host_i8(inp["q_idx"])
    rows = sample_rows(S, n_rows, seed)
    rows_t = torch.as_tensor(rows, device=DEV)
    osel = O.select_blocks(qi, summ, bs, K, rows)
    assert np.array_equal(host_i8(sel[:, :, rows_t]).astype(np.int32), osel), "selection differs on sampled rows"
    kk, vv = HostBf16(inp["k"]), HostBf16(inp["v"])
    _say(f"[backward {S}] oracle dq on {len(rows)} rows (worker processes)")
    rq, st = oracle_query_grads_pooled(inp, dout, osel, rows, bs)
    _say(f"[backward {S}] oracle dq: {st}")
    compare_grad(dq[:, rows_t], rq, f"{S} dq (sampled rows)")
    # the last block: only the queries inside it can keep it (candidates are
    # earlier blocks and the own one), so the oracle's selection of those
    # rows is all it needs; the other rows keep nothing here
    j = (S - 1) // bs
    tail = np.arange(j * bs, S)
    sel_full = np.full((B, G, S, K), -1, dtype=np.int32)
    sel_full[:, :, tail] = O.select_blocks(qi, summ, bs, K, tail)
    tail_t = torch.as_tensor(tail, device=DEV)
    gsel_tail = host_i8(sel[:, :, tail_t]).astype(np.int32)
    assert np.array_equal(gsel_tail, sel_full[:, :, tail]), "selection differs on the last block's rows"

    class Tail:
        """Rows [j * bs, S) of a [B, S, Hq, D] tensor, indexed by absolute row."""
        def __init__(self, t):
            self.h = t[:, j * bs:].to("cpu")
            self.shape = tuple(t.shape)

        def __getitem__(self, idx):
            b, t, hs = idx
            return self.h[b, t - j * bs, hs].float().numpy()

    _say(f"[backward {S}] oracle dk, dv of block {j}, group {g}")
    _, rk, rv = O.backward(Tail(inp["q"]), kk, vv, Tail(dout), sel_full, bs, rows=[], kv_blocks=[j], groups=[g])
    nt = S - j * bs  # keys of the (possibly ragged) last block
    compare_grad(dk[:, g, j * bs:], rk[:, g, 0, :nt], f"{S} dk block {j} group {g}")
    compare_grad(dv[:, g, j * bs:], rv[:, g, 0, :nt], f"{S} dv block {j} group {g}")


def test_backward_1m_passes_sampled_and_sums():
    """Prefill 1M (64 query heads, 8 groups, block 128, top_k 16) forward and
    backward; the backward's full workspace (about 275 GB) does not fit next
    to the tensors, so it runs in query passes.  dq on sampled rows and dk, dv
    of the last block of one group against the oracle; over every key, the
    closed-form sums of dv and dk."""
    w = get_workload("prefill_1m")
    S, bs, K = w.seq_len, w.block_size, w.top_k
    B, G = w.batch, w.n_kv_heads
    _say(f"[backward 1m] S={S}")
    inp = prefill_inputs(w, seed=43, device=DEV)
    dout = grad_output(w, seed=43, device=DEV)
    out, sel, lse = msa.msa_prefill_lse(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], bs, K)
    torch.cuda.synchronize()
    _free()
    dims = msa.make_dims(B, S, w.n_q_heads, G, bs, K)
    lo, hi = msa.msa_workspace_bytes(msa.MSA_OP_BACKWARD, dims)
    free, _ = torch.cuda.mem_get_info()
    _say(f"[backward 1m] workspace least {lo / 2**30:.1f} GiB, full {hi / 2**30:.1f} GiB, free {free / 2**30:.1f} GiB")
    assert hi > free, "the full workspace fits: the case would not run in passes"
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    dq, dk, dv = msa.msa_prefill_backward(inp["q"], inp["k"], inp["v"], out, dout, lse, sel, bs)
    t1.record()
    torch.cuda.synchronize()
    _say(f"[backward 1m] backward, with its allocations: {t0.elapsed_time(t1):.1f} ms")
    # a quarter of the way from the least to the full workspace: five passes,
    # the last one (32768 rows) planned with more histogram chunks than the
    # first ones
    ws = torch.empty(lo + (hi - lo) // 4, dtype=torch.uint8, device=DEV)
    rows = msa.msa_backward_pass_rows(dims, ws.numel())
    _say(f"[backward 1m] backward with a workspace of {ws.numel() / 2**30:.1f} GiB: passes of {rows} rows")
    assert 0 < rows < S and rows % 256 == 0 and -(-S // rows) >= 4
    dq4, dk4, dv4 = msa.msa_prefill_backward(inp["q"], inp["k"], inp["v"], out, dout, lse, sel, bs, workspace=ws)
    torch.cuda.synchronize()
    del ws, out, lse
    _free()
    assert torch.equal(dq4, dq), "1m: dq differs between pass sizes"
    _close_to_one_pass(dk4, dk, "1m dk (five passes vs two)")
    _close_to_one_pass(dv4, dv, "1m dv (five passes vs two)")
    del dq4, dk4, dv4
    _free()
    _check_long_backward(w, inp, dout, sel, dq, dk, dv, seed=43, g=3)
    del inp, dout, sel, dq, dk, dv
    _free()


def test_ragged_300k_forward_and_backward_passes():
    """300000 tokens (last block 96 tokens; four query chunks, the last one
    shorter): the forward on sampled rows, then the backward with a fifth of
    the way from the least to the full workspace (passes, the last one
    shorter), against the oracle."""
    from tests.helpers import compare_out, oracle_prefill_rows
    w = get_workload("prefill_1m", seq_len=300000)
    S, bs, K = w.seq_len, w.block_size, w.top_k
    _say(f"[ragged 300k] S={S}")
    inp = prefill_inputs(w, seed=47, device=DEV)
    dout = grad_output(w, seed=47, device=DEV)
    out, sel, lse = msa.msa_prefill_lse(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], bs, K)
    torch.cuda.synchronize()
    _free()
    rows = sample_rows(S, 48, 47)
    rows[-1] = S - 1
    rows_t = torch.as_tensor(rows, device=DEV)
    _say(f"[ragged 300k] oracle forward on {len(rows)} rows")
    _, osel, oout = oracle_prefill_rows(inp, w, rows)
    assert np.array_equal(host_i8(sel[:, :, rows_t]).astype(np.int32), osel), "selection differs on sampled rows"
    compare_out(out[:, rows_t], oout, "300k out (sampled rows)")
    ws, lo, hi = _pass_workspace(w, S, 0.2)
    _say(f"[ragged 300k] backward, workspace {ws.numel() / 2**30:.1f} GiB (least {lo / 2**30:.1f}, full {hi / 2**30:.1f})")
    dq, dk, dv = msa.msa_prefill_backward(inp["q"], inp["k"], inp["v"], out, dout, lse, sel, bs, workspace=ws)
    torch.cuda.synchronize()
    del ws, out, lse
    _free()
    _check_long_backward(w, inp, dout, sel, dq, dk, dv, seed=47, g=5)
    del inp, dout, sel, dq, dk, dv
    _free()
