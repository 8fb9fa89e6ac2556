"""Pins for the CPU oracle against things other than itself: hand-worked
values, brute force over subsets, closed forms and independent library
routines (torch's CPU attention).  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- pooling

def test_pool_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked.json"), encoding="utf-8"))
    k_idx = np.array(g["k_idx"], dtype=np.int8)[None, None]          # [1,1,S,di]
    s = O.pool_block_keys(k_idx, g["block_size"])
    assert s.dtype == np.int8
    assert s[0, 0].tolist() == g["summaries_expected"]


def test_pool_floor_not_truncation():
    # a block alternating -1 / 0 has mean -1/2: floor gives -1, truncation 0
    k = np.zeros((1, 1, 8, 4), dtype=np.int8)
    k[0, 0, 0::2] = -1
    assert (O.pool_block_keys(k, 8) == -1).all()
    # a constant block pools to that constant
    k = np.full((1, 1, 16, 3), -77, dtype=np.int8)
    assert (O.pool_block_keys(k, 16) == -77).all()
    # extremes do not overflow
    k = np.full((1, 1, 64, 2), -128, dtype=np.int8)
    assert (O.pool_block_keys(k, 64) == -128).all()
    k = np.full((1, 1, 64, 2), 127, dtype=np.int8)
    assert (O.pool_block_keys(k, 64) == 127).all()


@pytest.mark.parametrize("S,bs", [(40, 8), (37, 8), (5, 16), (64, 64)])
def test_pool_brute_force(S, bs):
    rng = _rng(S * 100 + bs)
    k = rng.integers(-128, 128, size=(2, 3, S, 5), dtype=np.int8)
    s = O.pool_block_keys(k, bs)
    nb = -(-S // bs)
    assert s.shape == (2, 3, nb, 5)
    for b in range(2):
        for g in range(3):
            for j in range(nb):
                toks = range(j * bs, min(S, (j + 1) * bs))
                for d in range(5):
                    total = sum(int(k[b, g, t, d]) for t in toks)
                    # math.floor on an exact Fraction-free ratio: use divmod
                    qf, rem = divmod(total, len(toks))   # Python floors toward -inf
                    assert rem >= 0
                    assert int(s[b, g, j, d]) == qf
                    assert qf <= total / len(toks) < qf + 1


# ---------------------------------------------------------------- selection

def test_select_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked.json"), encoding="utf-8"))
    summ = np.array(g["summaries_expected"], dtype=np.int8)
    for case in g["queries"]:
        qv = np.array(case["q_idx"], dtype=np.int8)
        c = case["t"] // g["block_size"]
        assert O.block_scores(qv, summ[:c]).tolist() == case["scores"]
        sel = O.select_row(qv, summ, case["t"], g["block_size"], g["top_k"])
        assert sel.tolist() == case["sel"], case


def _brute_force_selection(qv, summ, t, bs, top_k):
    """Top set as the maximum-score-sum subset; among equal sums the
    lexicographically smallest index tuple (which is what 'ties to the lower
    block index' amounts to).  Scores by explicit Python integer loops."""
    c = t // bs
    m = min(top_k - 1, c)
    score = [sum(int(qv[d]) * int(summ[j, d]) for d in range(len(qv))) for j in range(c)]
    best, best_sum = (), None
    for comb in itertools.combinations(range(c), m):     # lexicographic order
        s = sum(score[j] for j in comb)
        if best_sum is None or s > best_sum:
            best, best_sum = comb, s
    out = list(best) + [c]
    return out + [-1] * (top_k - len(out))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bs,top_k", [(4, 1), (4, 2), (2, 4), (8, 3)])
def test_select_brute_force(seed, bs, top_k):
    rng = _rng(1000 + seed)
    S, di = 10 * bs, 6
    # a narrow value range forces many score ties
    lo, hi = (-2, 3) if seed % 2 else (-64, 64)
    q_idx = rng.integers(lo, hi, size=(1, 1, S, di), dtype=np.int8)
    k_idx = rng.integers(lo, hi, size=(1, 1, S, di), dtype=np.int8)
    summ = O.pool_block_keys(k_idx, bs)
    sel = O.select_blocks(q_idx, summ, bs, top_k)
    for t in range(S):
        bf = _brute_force_selection(q_idx[0, 0, t], summ[0, 0], t, bs, top_k)
        assert sel[0, 0, t].tolist() == bf, (t, sel[0, 0, t], bf)


def test_select_special_cases():
    bs, S, di = 4, 40, 8
    rng = _rng(7)
    q_idx = rng.integers(-64, 64, size=(1, 2, S, di), dtype=np.int8)
    # all-equal summaries: every score ties, so the lowest indices win
    summ = np.full((1, 2, S // bs, di), 3, dtype=np.int8)
    sel = O.select_blocks(q_idx, summ, bs, 4)
    for t in range(S):
        c = t // bs
        exp = list(range(min(3, c))) + [c]
        assert sel[0, 0, t].tolist() == exp + [-1] * (4 - len(exp))
    # top_k = 1 keeps only the own block
    sel1 = O.select_blocks(q_idx, summ, bs, 1)
    assert (sel1[..., 0] == (np.arange(S) // bs)[None, None]).all()
    # a planted summary that matches the query strongly is always selected
    summ = rng.integers(-8, 8, size=(1, 1, S // bs, di), dtype=np.int8)
    qv = np.full(di, 100, dtype=np.int8)
    summ[0, 0, 2] = 100
    for t in range(3 * bs, S):
        assert 2 in O.select_row(qv, summ[0, 0], t, bs, 2)
    # group independence: group 1 sees only its own inputs
    q2 = q_idx.copy()
    q2[0, 1] = -q2[0, 1]
    summ2 = rng.integers(-64, 64, size=(1, 2, S // bs, di), dtype=np.int8)
    a = O.select_blocks(q_idx, summ2, bs, 3)
    b = O.select_blocks(q2, summ2, bs, 3)
    assert (a[:, 0] == b[:, 0]).all()


# ---------------------------------------------------------------- attention

def _rand_attention_inputs(seed, B, S, Hq, G, D):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, Hq, D, generator=g, dtype=torch.float64)
    k = torch.randn(B, G, S, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, G, S, D, generator=g, dtype=torch.float64)
    return q, k, v


def _sdpa(q, k, v, mask):
    """torch's CPU attention in fp64 with GQA expansion; q [B,S,Hq,D],
    k/v [B,G,S,D], mask bool [S,S] (True = attend)."""
    B, S, Hq, D = q.shape
    G = k.shape[1]
    r = Hq // G
    qh = q.permute(0, 2, 1, 3)                                 # [B,Hq,S,D]
    kh = k.repeat_interleave(r, dim=1)
    vh = v.repeat_interleave(r, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("S,bs,G,r", [(64, 8, 2, 4), (61, 8, 1, 8), (48, 16, 4, 1)])
def test_attention_equals_dense_when_all_blocks_selected(S, bs, G, r):
    B, D = 2, 16
    q, k, v = _rand_attention_inputs(S + bs, B, S, G * r, G, D)
    nb = -(-S // bs)
    rng = _rng(S)
    q_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    k_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    _, sel, out = O.prefill(q.numpy(), k.numpy(), v.numpy(), q_idx, k_idx, bs, nb)
    # every earlier block is selected, so this is dense causal attention
    for t in range(S):
        assert sorted(x for x in sel[0, 0, t] if x >= 0) == list(range(t // bs + 1))
    causal = torch.ones(S, S, dtype=torch.bool).tril()
    ref = _sdpa(q, k, v, causal)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-10)


def test_attention_own_block_only_is_block_diagonal():
    B, S, bs, G, r, D = 1, 40, 8, 2, 2, 8
    q, k, v = _rand_attention_inputs(5, B, S, G * r, G, D)
    rng = _rng(5)
    q_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    k_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    _, sel, out = O.prefill(q.numpy(), k.numpy(), v.numpy(), q_idx, k_idx, bs, 1)
    pos = torch.arange(S)
    mask = (pos[:, None] >= pos[None, :]) & (pos[:, None] // bs == pos[None, :] // bs)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask), rtol=0, atol=1e-10)


def test_attention_sparse_matches_masked_dense():
    """A sparse selection equals dense attention under the mask the selection
    implies (mask built here from the selection, attention by torch)."""
    B, S, bs, G, r, D, top_k = 1, 96, 8, 2, 4, 16, 4
    q, k, v = _rand_attention_inputs(11, B, S, G * r, G, D)
    rng = _rng(11)
    q_idx = rng.integers(-64, 64, size=(B, G, S, 16), dtype=np.int8)
    k_idx = rng.integers(-64, 64, size=(B, G, S, 16), dtype=np.int8)
    _, sel, out = O.prefill(q.numpy(), k.numpy(), v.numpy(), q_idx, k_idx, bs, top_k)
    for g in range(G):
        mask = torch.zeros(S, S, dtype=torch.bool)
        for t in range(S):
            for j in sel[0, g, t]:
                if j >= 0:
                    mask[t, j * bs:(j + 1) * bs] = True
        mask &= torch.ones(S, S, dtype=torch.bool).tril()
        ref = _sdpa(q[:, :, g * r:(g + 1) * r], k[:, g:g + 1], v[:, g:g + 1], mask)
        np.testing.assert_allclose(out[:, :, g * r:(g + 1) * r], ref, rtol=0, atol=1e-10)


def test_merge_of_any_partition_equals_one_softmax():
    """Closed form: the log-sum-exp merge of the states of any partition of
    the keys (per block, single keys, random groups) equals softmax attention
    over all of them."""
    rng = _rng(3)
    q = rng.standard_normal((6, 16))
    k = rng.standard_normal((40, 16))
    v = rng.standard_normal((40, 16))
    scale = 0.25
    ref = O.attend(q, k, v, scale)
    for parts in ([np.arange(40)], np.array_split(np.arange(40), 5), [np.array([i]) for i in range(40)],
                  np.array_split(rng.permutation(40), 7)):
        got = O.merge_states([O.partial_state(q, k[p], v[p], scale) for p in parts])
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # a state scaled consistently (o, l by e^d, m by -d) merges to the same result
    o, m, l = O.partial_state(q, k[:20], v[:20], scale)
    d = 3.0
    shifted = (o * np.exp(d), m - d, l * np.exp(d))
    got = O.merge_states([shifted, O.partial_state(q, k[20:], v[20:], scale)])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_weights_sum_to_one():
    # with every value row equal to c the output must be c exactly (up to
    # rounding): the weights of every row sum to 1
    B, S, bs, G, r, D = 1, 64, 8, 2, 4, 16
    q, k, _ = _rand_attention_inputs(3, B, S, G * r, G, D)
    c = np.linspace(-3, 3, D)
    v = np.broadcast_to(c, (B, G, S, D)).copy()
    rng = _rng(3)
    q_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    k_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    _, _, out = O.prefill(q.numpy() * 4.0, k.numpy(), v, q_idx, k_idx, bs, 3)
    assert np.abs(out - c).max() <= 1e-12


def test_attention_invariant_to_selection_order():
    B, S, bs, G, r, D, top_k = 1, 80, 8, 1, 4, 16, 5
    q, k, v = _rand_attention_inputs(9, B, S, G * r, G, D)
    rng = _rng(9)
    q_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    k_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    summ = O.pool_block_keys(k_idx, bs)
    rows = np.arange(S)
    sel = O.select_blocks(q_idx, summ, bs, top_k)
    perm = sel.copy()
    for t in range(S):
        rng.shuffle(perm[0, 0, t])
    a = O.attention_rows(q.numpy(), k.numpy(), v.numpy(), sel, rows, bs)
    b = O.attention_rows(q.numpy(), k.numpy(), v.numpy(), perm, rows, bs)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_first_query_returns_first_value():
    B, S, bs, G, r, D = 1, 16, 8, 2, 2, 8
    q, k, v = _rand_attention_inputs(2, B, S, G * r, G, D)
    rng = _rng(2)
    q_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    k_idx = rng.integers(-64, 64, size=(B, G, S, 8), dtype=np.int8)
    _, _, out = O.prefill(q.numpy(), k.numpy(), v.numpy(), q_idx, k_idx, bs, 2, rows=[0])
    for g in range(G):
        for h in range(g * r, (g + 1) * r):
            assert np.array_equal(out[0, 0, h], v.numpy()[0, g, 0])


def test_attention_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked.json"), encoding="utf-8"))
    a = g["attention"]
    vv = np.array(a["v"], dtype=np.float64)[None, None]               # [1,1,S,2]
    S = vv.shape[2]
    kk = np.zeros_like(vv)
    for case in a["cases"]:
        t = case["t"]
        keys = O.selected_keys(np.array(case["sel"]), t, g["block_size"], S)
        assert keys.tolist() == case["keys"]
        q_rows = np.ones((1, 1, 1, 2))
        sel = np.array(case["sel"], dtype=np.int32)[None, None, None]
        out = O.attention_rows(q_rows, kk, vv, sel, [t], g["block_size"])
        np.testing.assert_allclose(out[0, 0, 0], case["out"], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- decode

def test_decode_equals_last_prefill_row():
    B, L, bs, G, r, D, top_k = 2, 72, 8, 2, 4, 16, 4
    q, k, v = _rand_attention_inputs(21, B, L, G * r, G, D)
    rng = _rng(21)
    q_idx = rng.integers(-64, 64, size=(B, G, L, 8), dtype=np.int8)
    k_idx = rng.integers(-64, 64, size=(B, G, L, 8), dtype=np.int8)
    summ, sel, out = O.prefill(q.numpy(), k.numpy(), v.numpy(), q_idx, k_idx, bs, top_k,
                               rows=[L - 1])
    dsel, dout = O.decode(q.numpy()[:, L - 1], q_idx[:, :, L - 1], k.numpy(), v.numpy(), summ,
                          bs, top_k)
    assert np.array_equal(dsel, sel[:, :, 0])
    np.testing.assert_allclose(dout, out[:, 0], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- backward

def _sel_mask(sel, S, bs):
    """Attend mask [G, S, S] implied by a selection (built here, not by the
    oracle): keys of the kept blocks that are not after the query."""
    G = sel.shape[1]
    mask = torch.zeros(G, S, S, dtype=torch.bool)
    for g in range(G):
        for t in range(S):
            for j in sel[0, g, t]:
                if j >= 0:
                    mask[g, t, j * bs:(j + 1) * bs] = True
    return mask & torch.ones(S, S, dtype=torch.bool).tril()


def _autograd_grads(q, k, v, dout, mask):
    """dq, dk, dv of sum(dout * attention) by torch autograd in fp64 (B = 1),
    attention written as softmax of masked scores times v, per group."""
    S, Hq, D = q.shape[1:]
    G = k.shape[1]
    r = Hq // G
    q = q.clone().requires_grad_(True)
    k = k.clone().requires_grad_(True)
    v = v.clone().requires_grad_(True)
    outs = []
    for g in range(G):
        z = torch.einsum("shd,kd->hsk", q[0, :, g * r:(g + 1) * r], k[0, g]) / math.sqrt(D)
        z = z.masked_fill(~mask[g][None], float("-inf"))
        outs.append(torch.einsum("hsk,kd->shd", torch.softmax(z, dim=-1), v[0, g]))
    o = torch.cat(outs, dim=1)[None]
    (o * dout).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def _bwd_case(seed, S, bs, G, r, D, top_k, di=8):
    q, k, v = _rand_attention_inputs(seed, 1, S, G * r, G, D)
    dout = torch.randn(1, S, G * r, D, generator=torch.Generator().manual_seed(seed + 1), dtype=torch.float64)
    rng = _rng(seed)
    q_idx = rng.integers(-64, 64, size=(1, G, S, di), dtype=np.int8)
    k_idx = rng.integers(-64, 64, size=(1, G, S, di), dtype=np.int8)
    _, sel, _ = O.prefill(q.numpy(), k.numpy(), v.numpy(), q_idx, k_idx, bs, top_k)
    return q, k, v, dout, sel


def test_backward_equals_dense_sdpa_autograd_when_all_blocks_selected():
    """With every earlier block kept the gradients are those of dense causal
    GQA attention: torch's own attention, differentiated by autograd."""
    S, bs, G, r, D = 40, 8, 2, 2, 16
    q, k, v, dout, sel = _bwd_case(31, S, bs, G, r, D, top_k=5)
    dq, dk, dv = O.backward(q.numpy(), k.numpy(), v.numpy(), dout.numpy(), sel, bs)
    qq, kk, vv = (x.clone().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        qq.permute(0, 2, 1, 3), kk.repeat_interleave(r, dim=1), vv.repeat_interleave(r, dim=1), is_causal=True)
    (o.permute(0, 2, 1, 3) * dout).sum().backward()
    np.testing.assert_allclose(dq, qq.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk, kk.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dv, vv.grad.numpy(), rtol=0, atol=1e-10)


@pytest.mark.parametrize("S,bs,G,r,top_k", [(96, 8, 2, 4, 4), (61, 16, 1, 8, 2), (50, 8, 2, 1, 1)])
def test_backward_sparse_matches_masked_autograd(S, bs, G, r, top_k):
    q, k, v, dout, sel = _bwd_case(S + top_k, S, bs, G, r, 16, top_k)
    dq, dk, dv = O.backward(q.numpy(), k.numpy(), v.numpy(), dout.numpy(), sel, bs)
    rq, rk, rv = _autograd_grads(q, k, v, dout, _sel_mask(sel, S, bs))
    np.testing.assert_allclose(dq, rq, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk, rk, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dv, rv, rtol=0, atol=1e-10)


def test_backward_finite_differences():
    """Central differences of sum(dout * O) through the oracle's own forward,
    on every input element of a tiny case."""
    S, bs, G, r, D, top_k = 12, 4, 1, 2, 4, 2
    q, k, v, dout, sel = _bwd_case(7, S, bs, G, r, D, top_k)
    q, k, v, dout = (x.numpy() for x in (q, k, v, dout))
    dq, dk, dv = O.backward(q, k, v, dout, sel, bs)

    def loss(qx, kx, vx):
        return float((O.attention_rows(qx, kx, vx, sel, np.arange(S), bs) * dout).sum())

    h = 1e-6
    for which, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(which)
            args_p[pos], args_m[pos] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7)


def test_backward_sums_over_keys():
    """Closed forms: the softmax weights of a row sum to 1, so the dv rows of
    a group sum to the dout rows of its heads; the score gradients of a row
    sum to 0, so the dk rows of a group sum to 0."""
    S, bs, G, r, D, top_k = 80, 8, 2, 4, 8, 3
    q, k, v, dout, sel = _bwd_case(17, S, bs, G, r, D, top_k)
    _, dk, dv = O.backward(q.numpy(), k.numpy(), v.numpy(), dout.numpy(), sel, bs)
    d = dout.numpy()
    for g in range(G):
        np.testing.assert_allclose(dv[0, g].sum(axis=0), d[0, :, g * r:(g + 1) * r].sum(axis=(0, 1)), atol=1e-10)
        np.testing.assert_allclose(dk[0, g].sum(axis=0), 0.0, atol=1e-10)


def test_backward_rows_and_blocks_subsets():
    """Restricting the rows or the key blocks returns the same values."""
    S, bs, G, r, D, top_k = 72, 8, 2, 2, 8, 3
    q, k, v, dout, sel = _bwd_case(23, S, bs, G, r, D, top_k)
    q, k, v, dout = (x.numpy() for x in (q, k, v, dout))
    dq, dk, dv = O.backward(q, k, v, dout, sel, bs)
    rows, blocks = [0, 9, 40, 71], [0, 4, 8]
    sq, sk, sv = O.backward(q, k, v, dout, sel, bs, rows=rows, kv_blocks=blocks)
    np.testing.assert_array_equal(sq, dq[:, rows])
    gq, gk, gv = O.backward(q, k, v, dout, sel, bs, rows=rows, kv_blocks=blocks, groups=[1])
    np.testing.assert_array_equal(gq[:, :, r:], sq[:, :, r:])
    np.testing.assert_array_equal(gk[:, 1], sk[:, 1])
    assert not gq[:, :, :r].any() and not gk[:, 0].any() and not gv[:, 0].any()
    for i, j in enumerate(blocks):
        np.testing.assert_allclose(sk[:, :, i], dk[:, :, j * bs:(j + 1) * bs], rtol=0, atol=1e-14)
        np.testing.assert_allclose(sv[:, :, i], dv[:, :, j * bs:(j + 1) * bs], rtol=0, atol=1e-14)
    # no rows, or no blocks
    eq, ek, ev = O.backward(q, k, v, dout, sel, bs, rows=[], kv_blocks=[4])
    assert eq.shape == (1, 0, G * r, D)
    np.testing.assert_allclose(ek[:, :, 0], dk[:, :, 32:40], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ev[:, :, 0], dv[:, :, 32:40], rtol=0, atol=1e-14)
    fq, fk, _ = O.backward(q, k, v, dout, sel, bs, rows=[3, 50], kv_blocks=[])
    np.testing.assert_array_equal(fq, dq[:, [3, 50]])
    assert fk.shape == (1, G, 0, bs, D)


def test_query_grad_rows_matches_masked_autograd():
    """dq of a few rows alone, from the rows' own selection, against autograd
    of masked attention over every row."""
    S, bs, G, r, D, top_k = 70, 8, 2, 3, 16, 3
    q, k, v, dout, sel = _bwd_case(47, S, bs, G, r, D, top_k)
    rq, _, _ = _autograd_grads(q, k, v, dout, _sel_mask(sel, S, bs))
    rows = [0, 7, 8, 33, 69]
    dq = O.query_grad_rows(q.numpy()[:, rows], k.numpy(), v.numpy(), dout.numpy()[:, rows], sel[:, :, rows], rows,
                           bs)
    np.testing.assert_allclose(dq, rq[:, rows], rtol=0, atol=1e-10)


def test_lse_against_torch_logsumexp():
    S, bs, G, r, D, top_k = 64, 8, 2, 2, 16, 3
    q, k, v, dout, sel = _bwd_case(41, S, bs, G, r, D, top_k)
    lse = O.lse_rows(q.numpy(), k.numpy(), v.numpy(), sel, np.arange(S), bs)
    mask = _sel_mask(sel, S, bs)
    for g in range(G):
        z = torch.einsum("shd,kd->hsk", q[0, :, g * r:(g + 1) * r], k[0, g]) / math.sqrt(D)
        ref = torch.logsumexp(z.masked_fill(~mask[g][None], float("-inf")), dim=-1).T.numpy()
        np.testing.assert_allclose(lse[0, :, g * r:(g + 1) * r], ref, rtol=0, atol=1e-12)
    # the first query sees only key 0
    np.testing.assert_allclose(lse[0, 0], [q[0, 0, h].dot(k[0, h // r, 0]).item() / math.sqrt(D) for h in range(G * r)],
                               atol=1e-12)


# ---------------------------------------------------------------- bf16 rounding

def test_round_to_bf16_matches_torch_on_fp32_values():
    rng = _rng(4)
    x = rng.standard_normal(20000).astype(np.float32) * 10.0
    # add exact halfway cases between neighbouring bf16 values
    base = torch.randn(1000, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    bits = base.view(torch.int16).to(torch.int32)
    half = ((bits << 16) | 0x8000).to(torch.int32).view(torch.float32).numpy()
    x = np.concatenate([x, half, np.array([0.0, -0.0, 1.0, -2.5], np.float32)])
    ours = O.round_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    assert math.isclose(O.round_to_bf16(np.array([1.0 + 2 ** -9]))[0], 1.0)      # tie -> even
    assert math.isclose(O.round_to_bf16(np.array([1.0 + 3 * 2 ** -9]))[0], 1.0 + 2 ** -7)
