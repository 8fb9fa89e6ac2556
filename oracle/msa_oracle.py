"""CPU oracle for MiniMax Sparse Attention (MSA) -- TEST INFRASTRUCTURE ONLY.

Plain, slow, single-threaded NumPy.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the library never does.  It
shares no code, constants or helpers with the HIP path.

What it computes (the pages' description, then this library's fixed reading
of what the pages leave open):

* MSA is grouped-query attention split into two branches: an index branch
  that scores KV blocks cheaply and lets every GQA group pick its own top-k
  set, and a main branch that runs exact attention over the picked blocks
  only ("深度解析 MiniMax-M3：稀疏注意力机制、基准测试与 API 集成指南",
  section "架构核心：MoE 与 MSA 的深度融合", items 1 and 2; the flowchart of
  the wiki.500nian.com digest of "MiniMax M3 Review: 1M Tokens, 15X Faster AI
  Agents", nodes "Index Branch" and "Main Branch").
* The ranking uses no exponentials: integer scores are compared directly
  (same digest, flowchart node "exp-free Top-k"; the n1n.ai article,
  paragraph "专业建议").
* Attention itself is softmax(q k^T / sqrt(d)) v (chenxutan.com guide,
  section 2.1, the attention formula).

Fixed reading of the index branch (the pages give no formula):
  - every token has one int8 index query and one int8 index key per group,
    of width d_i = 64;
  - a block's summary key is the floor (toward -inf) of the integer mean of
    its tokens' index keys; a ragged last block divides by its own count;
  - a block's score for a query is the exact integer dot product of the
    query's index vector with the summary;
  - only blocks strictly before the query's own block are ranked, by score
    descending, ties to the lower block index; the best top_k - 1 are kept
    (all of them when fewer exist) and the query's own block is always added;
  - the selection is reported ascending, padded with -1 to top_k entries;
  - query head h belongs to group h // (Hq / G);
  - attention runs one softmax over every key of the selected blocks that is
    not after the query (key position <= query position), scale 1/sqrt(D).

Floating point is fp64 throughout; the inputs are bf16 values carried
exactly in fp64.  The decode step is the same rule for the last position of
a cache.
"""
import math

import numpy as np


# --------------------------------------------------------------------------
# index branch
# --------------------------------------------------------------------------

def pool_block_keys(k_idx: np.ndarray, block_size: int) -> np.ndarray:
    """Block summary keys: floor of the integer mean of each block's keys.

    k_idx: int8 [B, G, S, di]  ->  int8 [B, G, nb, di], nb = ceil(S / bs).
    """
    B, G, S, di = k_idx.shape
    nb = -(-S // block_size)
    out = np.empty((B, G, nb, di), dtype=np.int64)
    for j in range(nb):
        t0, t1 = j * block_size, min(S, (j + 1) * block_size)
        total = k_idx[:, :, t0:t1, :].astype(np.int64).sum(axis=2)
        out[:, :, j, :] = np.floor_divide(total, t1 - t0)
    return out.astype(np.int8)


def block_scores(q_vec: np.ndarray, summaries: np.ndarray) -> np.ndarray:
    """Exact integer dot products of one index query with block summaries."""
    return summaries.astype(np.int64) @ q_vec.astype(np.int64)


def select_row(q_vec: np.ndarray, summaries: np.ndarray, t: int, block_size: int,
               top_k: int) -> np.ndarray:
    """Selected blocks of one (query position t, group): int32 [top_k]."""
    c = t // block_size
    scores = block_scores(q_vec, summaries[:c])
    cand = np.arange(c, dtype=np.int64)
    # primary key: score descending; secondary key: block index ascending
    order = np.lexsort((cand, -scores))
    taken = np.sort(cand[order[:min(top_k - 1, c)]])
    sel = np.full(top_k, -1, dtype=np.int32)
    sel[:len(taken)] = taken
    sel[len(taken)] = c
    return sel


def select_blocks(q_idx: np.ndarray, summaries: np.ndarray, block_size: int, top_k: int,
                  rows=None) -> np.ndarray:
    """Selections for every (b, g) and query row.

    q_idx: int8 [B, G, S, di]; summaries: int8 [B, G, nb, di];
    rows: query positions (default: all).  Returns int32 [B, G, len(rows), top_k].
    """
    B, G, S, _ = q_idx.shape
    rows = np.arange(S) if rows is None else np.asarray(rows)
    out = np.empty((B, G, len(rows), top_k), dtype=np.int32)
    for b in range(B):
        for g in range(G):
            for i, t in enumerate(rows):
                out[b, g, i] = select_row(q_idx[b, g, t], summaries[b, g], int(t), block_size, top_k)
    return out


# --------------------------------------------------------------------------
# main branch
# --------------------------------------------------------------------------

def selected_keys(sel_row: np.ndarray, t: int, block_size: int, seq_len: int) -> np.ndarray:
    """Key positions a query attends to: all tokens of its selected blocks
    that are not after the query."""
    keys = []
    for j in sel_row:
        if j < 0:
            continue
        s0, s1 = int(j) * block_size, min(seq_len, (int(j) + 1) * block_size)
        keys.append(np.arange(s0, s1))
    keys = np.concatenate(keys)
    return keys[keys <= t]


def attend(q_rows: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q k^T * scale) v for query rows [n, D] over keys [m, D]."""
    z = (q_rows @ k_sel.T) * scale
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ v_sel


def partial_state(q_rows: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float):
    """Unnormalised softmax state of query rows [n, D] over a subset of their
    keys [m, D]: (o = sum_s e^(z_s - m) v_s, m = max_s z_s, l = sum_s
    e^(z_s - m)), z = q.k * scale."""
    z = (q_rows @ k_sel.T) * scale
    m = z.max(axis=1)
    w = np.exp(z - m[:, None])
    return w @ v_sel, m, w.sum(axis=1)


def merge_states(states) -> np.ndarray:
    """Log-sum-exp combination of the states of a partition of the attended
    keys: O = sum_i e^(m_i - M) o_i / sum_i e^(m_i - M) l_i, M = max_i m_i.
    Equals one softmax over all the keys (the identity the main branch's
    per-block partials rely on)."""
    M = np.max([m for _, m, _ in states], axis=0)
    num = sum(np.exp(m - M)[:, None] * o for o, m, _ in states)
    den = sum(np.exp(m - M) * l for _, m, l in states)
    return num / den[:, None]

def attention_rows(q_rows, k, v, sel, rows, block_size: int, scale=None) -> np.ndarray:
    """MSA main-branch output for the given query rows.

    q_rows: [B, len(rows), Hq, D]; k, v: [B, G, S, D]; sel: int32
    [B, G, len(rows), top_k].  Any float dtype that holds the bf16 inputs
    exactly (fp32 or fp64); every gathered operand is widened to fp64.
    Returns float64 [B, len(rows), Hq, D].
    """
    B, R, Hq, D = q_rows.shape
    G, S = k.shape[1], k.shape[2]
    r = Hq // G
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.empty((B, R, Hq, D), dtype=np.float64)
    for b in range(B):
        for i, t in enumerate(np.asarray(rows)):
            for g in range(G):
                keys = selected_keys(sel[b, g, i], int(t), block_size, S)
                out[b, i, g * r:(g + 1) * r] = attend(
                    q_rows[b, i, g * r:(g + 1) * r].astype(np.float64),
                    k[b, g, keys].astype(np.float64), v[b, g, keys].astype(np.float64), scale)
    return out


def prefill(q, k, v, q_idx, k_idx, block_size: int, top_k: int, rows=None, scale=None):
    """Whole prefill for the given rows (default all): (summaries, sel, out)."""
    S = q.shape[1]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    summaries = pool_block_keys(k_idx, block_size)
    sel = select_blocks(q_idx, summaries, block_size, top_k, rows)
    out = attention_rows(q[:, rows], k, v, sel, rows, block_size, scale)
    return summaries, sel, out


def decode(q, q_idx, k_cache, v_cache, summaries, block_size: int, top_k: int, scale=None):
    """One decode step for the query at the last cache position L - 1.

    q: [B, Hq, D]; q_idx: int8 [B, G, di]; caches [B, G, L, D] (fp32 or fp64);
    summaries: int8 [B, G, nb, di].  Returns (sel int32 [B, G, top_k],
    out float64 [B, Hq, D]).
    """
    B, Hq, D = q.shape
    G, L = k_cache.shape[1], k_cache.shape[2]
    r = Hq // G
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    t = L - 1
    sel = np.empty((B, G, top_k), dtype=np.int32)
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for g in range(G):
            sel[b, g] = select_row(q_idx[b, g], summaries[b, g], t, block_size, top_k)
            keys = selected_keys(sel[b, g], t, block_size, L)
            out[b, g * r:(g + 1) * r] = attend(
                q[b, g * r:(g + 1) * r].astype(np.float64), k_cache[b, g, keys].astype(np.float64),
                v_cache[b, g, keys].astype(np.float64), scale)
    return sel, out


# --------------------------------------------------------------------------
# main branch, training: log-sum-exp and gradients with the selection fixed
# --------------------------------------------------------------------------
#
# The pages report ablations of trained MSA models and a training cost
# (wiki.500nian.com digest of "MiniMax M3 Review", the ablation paragraph;
# devpress.csdn.net article, section "M3的技术局限与改进方向", third
# limitation) but print no backward formula.  The reading here: the index
# branch is integer arithmetic and carries no gradient, so the selection is a
# constant of the backward pass, and the gradients are those of the forward
# definition above -- one softmax over the attended keys -- by the chain rule.

def lse_rows(q_rows, k, v, sel, rows, block_size: int, scale=None) -> np.ndarray:
    """Natural log-sum-exp of the scaled scores q.k * scale over the keys a
    query row attends to: [B, len(rows), Hq] float64."""
    B, R, Hq, D = q_rows.shape
    G, S = k.shape[1], k.shape[2]
    r = Hq // G
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.empty((B, R, Hq), dtype=np.float64)
    for b in range(B):
        for i, t in enumerate(np.asarray(rows)):
            for g in range(G):
                keys = selected_keys(sel[b, g, i], int(t), block_size, S)
                z = (q_rows[b, i, g * r:(g + 1) * r].astype(np.float64) @ k[b, g, keys].astype(np.float64).T) * scale
                zm = z.max(axis=1, keepdims=True)
                out[b, i, g * r:(g + 1) * r] = (zm + np.log(np.exp(z - zm).sum(axis=1, keepdims=True)))[:, 0]
    return out


def _query_grads(qh, ks, vs, doh, scale):
    """Gradients of sum(do * o) for o = softmax(qh ks^T * scale) vs, for the r
    query heads of one token over its m attended keys.

    qh, doh: [r, D]; ks, vs: [m, D].  With w the softmax weights [r, m]:
      dv = w^T do;  dw = do vs^T;  dz = w * (dw - rowsum(w * dw));
      dq = scale dz ks;  dk = scale dz^T qh.
    """
    z = (qh @ ks.T) * scale
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=1, keepdims=True)
    dw = doh @ vs.T
    dz = w * (dw - (w * dw).sum(axis=1, keepdims=True))
    return scale * (dz @ ks), scale * (dz.T @ qh), w.T @ doh


def backward(q, k, v, dout, sel, block_size: int, scale=None, rows=None, kv_blocks=None, groups=None):
    """Gradients of sum(dout * O) with respect to q, k and v, O being the
    main-branch output of every query row and the selection sel
    [B, G, S, top_k] held fixed.

    q, dout: [B, S, Hq, D]; k, v: [B, G, S, D] (fp32 or fp64 holding the bf16
    inputs).  Returns float64 (dq [B, len(rows), Hq, D] for the query rows
    `rows` (default all), dk, dv [B, G, len(kv_blocks), block_size, D] for
    the key blocks `kv_blocks` (default all blocks, then reshaped to
    [B, G, S, D])).  dk and dv of a block sum the contributions of every
    query whose selection holds it.  `groups` (default all) limits the work
    to those GQA groups; the other groups' entries stay zero.
    """
    B, S, Hq, D = q.shape
    G = k.shape[1]
    r = Hq // G
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    nb = -(-S // block_size)
    all_blocks = kv_blocks is None
    blocks = np.arange(nb) if all_blocks else np.asarray(kv_blocks, dtype=np.int64)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    row_pos = {int(t): i for i, t in enumerate(rows)}
    blk_pos = {int(j): i for i, j in enumerate(blocks)}
    dq = np.zeros((B, len(rows), Hq, D), dtype=np.float64)
    dkb = np.zeros((B, G, len(blocks), block_size, D), dtype=np.float64)
    dvb = np.zeros_like(dkb)
    for b in range(B):
        for g in (range(G) if groups is None else groups):
            hs = slice(g * r, (g + 1) * r)
            # the rows that matter: those asked for and those that kept one
            # of the asked blocks (every other row contributes nothing)
            visit = np.isin(sel[b, g], blocks).any(axis=1)
            visit[rows] = True
            for t in np.flatnonzero(visit):
                t = int(t)
                keys = selected_keys(sel[b, g, t], t, block_size, S)
                gq, gk, gv = _query_grads(q[b, t, hs].astype(np.float64), k[b, g, keys].astype(np.float64),
                                          v[b, g, keys].astype(np.float64), dout[b, t, hs].astype(np.float64),
                                          scale)
                if t in row_pos:
                    dq[b, row_pos[t], hs] = gq
                for i, key in enumerate(keys):
                    j = int(key) // block_size
                    if j in blk_pos:
                        dkb[b, g, blk_pos[j], int(key) % block_size] += gk[i]
                        dvb[b, g, blk_pos[j], int(key) % block_size] += gv[i]
    if all_blocks:
        dkb = dkb.reshape(B, G, nb * block_size, D)[:, :, :S]
        dvb = dvb.reshape(B, G, nb * block_size, D)[:, :, :S]
    return dq, dkb, dvb


def query_grad_rows(q_rows, k, v, dout_rows, sel, rows, block_size: int, scale=None):
    """dq of the given query rows alone, for long sequences: a row's query
    gradient depends only on its own q and dout and on the keys it attends
    to, so no other row is visited.

    q_rows, dout_rows: [B, len(rows), Hq, D]; k, v: [B, G, S, D] (any
    indexable holding the bf16 inputs); sel: int32 [B, G, len(rows), top_k].
    Returns float64 [B, len(rows), Hq, D], equal to backward(..., rows=rows)'s dq.
    """
    B, R, Hq, D = q_rows.shape
    G, S = k.shape[1], k.shape[2]
    r = Hq // G
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dq = np.empty((B, R, Hq, D), dtype=np.float64)
    for b in range(B):
        for i, t in enumerate(np.asarray(rows)):
            for g in range(G):
                hs = slice(g * r, (g + 1) * r)
                keys = selected_keys(sel[b, g, i], int(t), block_size, S)
                dq[b, i, hs], _, _ = _query_grads(q_rows[b, i, hs].astype(np.float64),
                                                  k[b, g, keys].astype(np.float64),
                                                  v[b, g, keys].astype(np.float64),
                                                  dout_rows[b, i, hs].astype(np.float64), scale)
    return dq


# --------------------------------------------------------------------------
# output rounding used by the comparison
# --------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned
    as fp64.  bf16 keeps 8 significant bits; values are assumed finite and
    inside bf16's normal range or zero."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
