"""The allocation-free decode entry point (msa_decode_noalloc, fixed
per-device scratch) against msa_decode (caller workspace) through the C ABI:
two calls in a row, the second on a smaller input, each bit-equal to
msa_decode on the same input (same kernels), selection included; the first
is also held to the oracle's tolerance."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_33_amd as msa
from oracle import msa_oracle as O
from synth import decode_inputs, get_workload
from tests.helpers import HostBf16, compare_out, host_f32, host_i8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(w, L, B, seed):
    print(f"[decode noalloc] L={L} B={B} {w}", flush=True)
    sys.stdout.flush()
    inp = decode_inputs(w, seed=seed, device=DEV, seq_len=L, batch=B)
    bk = msa.msa_pool_block_keys(inp["k_idx_cache"], w.block_size)
    ref, rsel = msa.msa_decode(inp["q"], inp["q_idx"], inp["k_cache"], inp["v_cache"], bk, w.block_size, w.top_k,
                               return_sel=True)
    out = torch.empty_like(inp["q"])
    sel = torch.full((B, w.n_kv_heads, w.top_k), -7, dtype=torch.int32, device=DEV)
    msa.msa_decode_noalloc(inp["q"], inp["q_idx"], inp["k_cache"], inp["v_cache"], bk, w.block_size, w.top_k,
                           out, sel=sel)
    torch.cuda.synchronize()
    assert torch.equal(sel, rsel), "selection differs from msa_decode"
    assert torch.equal(out, ref), "output differs from msa_decode"
    return inp, bk, out, sel


def test_decode_noalloc_two_calls_second_smaller():
    w = get_workload("decode_b16_256k")
    inp, bk, out, sel = _case(w, 100000, 8, seed=901)
    summ = O.pool_block_keys(host_i8(inp["k_idx_cache"]), w.block_size)
    osel, oout = O.decode(host_f32(inp["q"]), host_i8(inp["q_idx"]), HostBf16(inp["k_cache"]),
                          HostBf16(inp["v_cache"]), summ, w.block_size, w.top_k)
    assert np.array_equal(host_i8(sel).astype(np.int32), osel)
    compare_out(out, oout, "decode noalloc L=100000")
    del inp, bk, out, sel
    # a smaller second call, with other heads and top_k: it reuses the same
    # scratch array, whose contents from the first call must not matter
    w2 = get_workload("decode_b16_256k", n_q_heads=16, n_kv_heads=4, block_size=64, top_k=6)
    _case(w2, 3000, 2, seed=902)
    # and no sel pointer: the selection then goes to the scratch as well
    inp3 = decode_inputs(w2, seed=903, device=DEV, seq_len=777, batch=1)
    bk3 = msa.msa_pool_block_keys(inp3["k_idx_cache"], w2.block_size)
    ref3 = msa.msa_decode(inp3["q"], inp3["q_idx"], inp3["k_cache"], inp3["v_cache"], bk3, w2.block_size, w2.top_k)
    out3 = torch.empty_like(inp3["q"])
    msa.msa_decode_noalloc(inp3["q"], inp3["q_idx"], inp3["k_cache"], inp3["v_cache"], bk3, w2.block_size,
                           w2.top_k, out3)
    torch.cuda.synchronize()
    assert torch.equal(out3, ref3)


def test_decode_noalloc_rejects_oversized_shape():
    """65536 one-token sequences x 8 groups: their selections (33.5 MB) do
    not fit the fixed scratch; the call is refused before any launch."""
    w = get_workload("decode_b16_256k", n_q_heads=8, n_kv_heads=8, top_k=16)
    q = torch.zeros((65536, 8, 128), dtype=torch.bfloat16, device=DEV)
    qi = torch.zeros((65536, 8, 64), dtype=torch.int8, device=DEV)
    kc = torch.zeros((65536, 8, 1, 128), dtype=torch.bfloat16, device=DEV)
    bk = torch.zeros((65536, 8, 1, 64), dtype=torch.int8, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_decode_noalloc(q, qi, kc, kc, bk, w.block_size, w.top_k, out)
    assert e.value.code == msa._lib.MSA_ERR_SCRATCH
