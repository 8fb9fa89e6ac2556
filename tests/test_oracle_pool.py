"""The oracle's worker-process drivers (oracle/pool.py) return what the
oracle's own functions return when called directly: selections bit-equal,
values equal up to the summation order of multi-threaded fp64 BLAS calls in
this process against one-thread ones in the workers (relative 1e-12).  Two
worker processes, so the process path runs; small shapes with a ragged last
block and two batch entries."""
import numpy as np
import torch

from oracle import msa_oracle as O
from oracle import pool as P
from synth import get_workload, grad_output, prefill_inputs
from tests.helpers import host_bits, host_f32, host_i8

W = get_workload("tiny_2k", batch=2, n_q_heads=4, n_kv_heads=2, block_size=32, top_k=5)
S = 300


def _inputs():
    inp = prefill_inputs(W, seed=7, device="cpu", seq_len=S)
    dout = grad_output(W, seed=7, device="cpu", seq_len=S)
    return inp, dout


def _close(a, b):
    scale = max(float(np.abs(b).max()), 1e-30)
    assert float(np.abs(a - b).max()) <= 1e-12 * scale


def test_pool_prefill_rows_match_the_oracle():
    inp, _ = _inputs()
    rows = np.array([0, 31, 32, 100, 257, S - 1])
    rt = torch.as_tensor(rows)
    summ, sel, out, st = P.prefill_rows(host_bits(inp["q"][:, rt]), host_bits(inp["k"]), host_bits(inp["v"]),
                                        host_i8(inp["q_idx"]), host_i8(inp["k_idx"]), rows, W.block_size, W.top_k,
                                        workers=2)
    assert st["rows"] == len(rows)
    osumm = O.pool_block_keys(host_i8(inp["k_idx"]), W.block_size)
    osel = O.select_blocks(host_i8(inp["q_idx"]), osumm, W.block_size, W.top_k, rows)
    oout = O.attention_rows(host_f32(inp["q"][:, rt]), host_f32(inp["k"]), host_f32(inp["v"]), osel, rows,
                            W.block_size)
    assert np.array_equal(summ, osumm) and np.array_equal(sel, osel)
    # the pool stores bf16-rounded outputs
    assert np.array_equal(out, O.round_to_bf16(oout).astype(np.float32))


def test_pool_query_grad_rows_match_the_oracle():
    inp, dout = _inputs()
    rows = np.array([1, 33, 64, 200, S - 1])
    rt = torch.as_tensor(rows)
    summ = O.pool_block_keys(host_i8(inp["k_idx"]), W.block_size)
    sel = O.select_blocks(host_i8(inp["q_idx"]), summ, W.block_size, W.top_k, rows)
    dq, st = P.query_grad_rows(host_bits(inp["q"][:, rt]), host_bits(dout[:, rt]), host_bits(inp["k"]),
                               host_bits(inp["v"]), sel, rows, W.block_size, workers=2)
    assert st["rows"] == len(rows)
    ref = O.query_grad_rows(host_f32(inp["q"][:, rt]), host_f32(inp["k"]), host_f32(inp["v"]), host_f32(dout[:, rt]),
                            sel, rows, W.block_size)
    _close(dq, ref)


def test_pool_kv_grad_pairs_match_the_oracle():
    inp, dout = _inputs()
    summ = O.pool_block_keys(host_i8(inp["k_idx"]), W.block_size)
    sel = O.select_blocks(host_i8(inp["q_idx"]), summ, W.block_size, W.top_k)
    nb = -(-S // W.block_size)
    pairs = [(0, 0), (3, 1), (nb - 1, 1)]  # the last block is ragged (300 = 9 * 32 + 12)
    dk, dv, st = P.kv_grad_pairs(host_bits(inp["q"]), host_bits(dout), host_bits(inp["k"]), host_bits(inp["v"]),
                                 sel, pairs, W.block_size, workers=2)
    assert st["pairs"] == len(pairs)
    _, rk, rv = O.backward(host_f32(inp["q"]), host_f32(inp["k"]), host_f32(inp["v"]), host_f32(dout), sel,
                           W.block_size, kv_blocks=[j for j, _ in pairs])
    for i, (j, g) in enumerate(pairs):
        _close(dk[:, i], rk[:, g, i])
        _close(dv[:, i], rv[:, g, i])
    # rows past the sequence end in the ragged last block stay zero
    tail = S - (nb - 1) * W.block_size
    assert not dk[:, 2, tail:].any() and not dv[:, 2, tail:].any()
