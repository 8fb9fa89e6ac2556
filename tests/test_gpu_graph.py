"""HIP graph capture of the library's calls (through torch.cuda.graph): a
serving loop records a decode or a generation step once and replays it.
The calls enqueue kernels only (no memset, copy or synchronisation), so a
capture records them as they are; each test replays the graph several
times, with eager work and a synchronisation between replays, and checks
every replay bit for bit against the eager call on the same inputs."""
import pytest
import torch

import block_sparse_attention_33_amd as msa
from synth import decode_inputs, get_workload, prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 3


def _say(*a):
    print(*a, flush=True)


def _capture(fn):
    """fn() run once eagerly on a side stream (first-call set-up), then
    captured into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _eager_noise():
    # unrelated eager work between replays
    x = torch.randn(1 << 20, device=DEV)
    return float((x * x).mean())


def _check_replays(g, outs, refs, before=None):
    for i in range(REPLAYS):
        for o in outs:
            o.zero_()
        if before is not None:
            before()
        _eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {i} differs from the eager call"


def _decode_ws(dims_fn):
    lo, _ = msa.msa_workspace_bytes(msa.MSA_OP_DECODE, dims_fn)
    return torch.empty(max(lo, 256), dtype=torch.uint8, device=DEV)


def test_decode_graph_replays():
    w = get_workload("decode_b16_256k", n_q_heads=16, n_kv_heads=2, block_size=128, top_k=16)
    B, L = 4, 20000
    _say(f"[graph] decode B={B} L={L}")
    inp = decode_inputs(w, seed=13, device=DEV, seq_len=L, batch=B)
    bk = msa.msa_pool_block_keys(inp["k_idx_cache"], w.block_size)
    dims = msa.make_dims(B, L, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
    ws = _decode_ws(dims)
    out = torch.empty_like(inp["q"])
    sel = torch.empty((B, w.n_kv_heads, w.top_k), dtype=torch.int32, device=DEV)

    def call():
        msa.msa_decode(inp["q"], inp["q_idx"], inp["k_cache"], inp["v_cache"], bk, w.block_size, w.top_k, out=out,
                       sel=sel, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = (out.clone(), sel.clone())
    g = _capture(call)
    _check_replays(g, [out, sel], ref)


def test_decode_varlen_graph_replays():
    """A captured ragged decode replays with the lengths it was captured
    with (they travel in the captured kernel arguments)."""
    w = get_workload("decode_b16_256k", n_q_heads=8, n_kv_heads=2, block_size=64, top_k=8)
    lens, C = [5, 700, 3000, 12000], 12000
    B = len(lens)
    _say(f"[graph] decode varlen lengths={lens}")
    inp = decode_inputs(w, seed=17, device=DEV, seq_len=C, batch=B)
    bk, _ = msa.msa_decode_init_varlen(inp["k_idx_cache"], lens, w.block_size)
    dims = msa.make_dims(B, C, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
    ws = _decode_ws(dims)
    out = torch.empty_like(inp["q"])
    sel = torch.empty((B, w.n_kv_heads, w.top_k), dtype=torch.int32, device=DEV)

    def call():
        msa.msa_decode_varlen(inp["q"], inp["q_idx"], inp["k_cache"], inp["v_cache"], bk, lens, w.block_size,
                              w.top_k, out=out, sel=sel, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = (out.clone(), sel.clone())
    g = _capture(call)
    _check_replays(g, [out, sel], ref)


def test_decode_step_graph_replays():
    """The generation step (append + decode) captured once: before each
    replay the caches, summaries and open-block sums are reset to the state
    the eager step started from, and each replay leaves exactly the eager
    step's outputs and state."""
    w = get_workload("decode_b16_256k", n_q_heads=8, n_kv_heads=2, block_size=64, top_k=6)
    B, C, L = 3, 4096, 1000
    _say(f"[graph] decode step B={B} length={L}")
    tr = decode_inputs(w, seed=19, device=DEV, seq_len=C, batch=B)
    kc, vc, kidx = tr["k_cache"].clone(), tr["v_cache"].clone(), tr["k_idx_cache"].clone()
    kc[:, :, L - 1:] = 0
    vc[:, :, L - 1:] = 0
    bk, osum = msa.msa_decode_init(kidx, L - 1, w.block_size)
    qs = decode_inputs(w, seed=23, device=DEV, seq_len=1, batch=B)
    k_new = tr["k_cache"][:, :, L - 1].contiguous()
    v_new = tr["v_cache"][:, :, L - 1].contiguous()
    ki_new = tr["k_idx_cache"][:, :, L - 1].contiguous()
    dims = msa.make_dims(B, C, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
    ws = _decode_ws(dims)
    out = torch.empty_like(qs["q"])
    sel = torch.empty((B, w.n_kv_heads, w.top_k), dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    state = [kc, vc, osum, bk]
    start = [t.clone() for t in state]

    def reset():
        for t, s0 in zip(state, start):
            t.copy_(s0)

    def call():
        msa.msa_decode_step(qs["q"], qs["q_idx"], k_new, v_new, ki_new, kc, vc, osum, bk, L, w.block_size, w.top_k,
                            out=out, sel=sel, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = [out.clone(), sel.clone()] + [t.clone() for t in state]
    reset()
    torch.cuda.synchronize()
    g = _capture(call)
    _check_replays(g, [out, sel] + state, ref, before=reset)


def test_prefill_graph_replays():
    w = get_workload("tiny_2k", batch=2, n_q_heads=8, n_kv_heads=2, block_size=64, top_k=6)
    S = 5000
    _say(f"[graph] prefill B=2 S={S}")
    inp = prefill_inputs(w, seed=29, device=DEV, seq_len=S)
    dims = msa.make_dims(2, S, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
    lo, hi = msa.msa_workspace_bytes(msa.MSA_OP_PREFILL, dims)
    ws = torch.empty(hi, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(inp["q"])
    sel = torch.empty((2, w.n_kv_heads, S, w.top_k), dtype=torch.int32, device=DEV)

    def call():
        msa.msa_prefill(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], w.block_size, w.top_k, out=out,
                        sel=sel, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = (out.clone(), sel.clone())
    g = _capture(call)
    _check_replays(g, [out, sel], ref)


def test_generation_loop_graph_device_lengths():
    """A ragged generation loop captured once: the step reads its lengths
    from device memory, so each of 40 replays -- inputs copied into the
    captured buffers and the lengths advanced on the device before it --
    decodes the next position.  Every step's output and selection, and the
    caches, summaries and open sums at the end, are bit-equal to the same
    steps run eagerly with host lengths on a copy of the state."""
    w = get_workload("decode_b16_256k", n_q_heads=8, n_kv_heads=2, block_size=64, top_k=6)
    L0s, steps = [1, 63, 64, 500], 40
    B, C, bs, k = len(L0s), max(L0s) + steps + 8, w.block_size, w.top_k
    _say(f"[graph] generation loop L0={L0s} steps={steps}")
    tr = decode_inputs(w, seed=31, device=DEV, seq_len=C, batch=B)
    kc, vc = tr["k_cache"].clone(), tr["v_cache"].clone()
    for b, L0 in enumerate(L0s):
        kc[b, :, L0:] = 0
        vc[b, :, L0:] = 0
    bk, osum = msa.msa_decode_init_varlen(tr["k_idx_cache"], L0s, bs)
    ekc, evc, ebk, eos = kc.clone(), vc.clone(), bk.clone(), osum.clone()  # the eager copy
    lens = torch.tensor([L0 + 1 for L0 in L0s], dtype=torch.int32, device=DEV)
    qb = torch.empty((B, w.n_q_heads, 128), dtype=torch.bfloat16, device=DEV)
    qib = torch.empty((B, w.n_kv_heads, 64), dtype=torch.int8, device=DEV)
    knb = torch.empty((B, w.n_kv_heads, 128), dtype=torch.bfloat16, device=DEV)
    vnb = torch.empty_like(knb)
    kinb = torch.empty((B, w.n_kv_heads, 64), dtype=torch.int8, device=DEV)
    dims = msa.make_dims(B, C, w.n_q_heads, w.n_kv_heads, bs, k)
    ws = _decode_ws(dims)
    out = torch.empty_like(qb)
    sel = torch.empty((B, w.n_kv_heads, k), dtype=torch.int32, device=DEV)
    ar = torch.arange(B, device=DEV)

    def call():
        msa.msa_decode_step_varlen(qb, qib, knb, vnb, kinb, kc, vc, osum, bk, lens, bs, k, out=out, sel=sel,
                                   workspace=ws)

    # capture without running a step on the real state: the warm-up runs on
    # copies
    state = [kc, vc, osum, bk]
    saved = [t.clone() for t in state]
    g = _capture(call)
    for t, s0 in zip(state, saved):
        t.copy_(s0)
    for i in range(steps):
        hl = [L0 + i + 1 for L0 in L0s]
        pos = torch.tensor([x - 1 for x in hl], device=DEV)
        qs = decode_inputs(w, seed=900 + i, device=DEV, seq_len=1, batch=B)
        qb.copy_(qs["q"])
        qib.copy_(qs["q_idx"])
        knb.copy_(tr["k_cache"][ar, :, pos])
        vnb.copy_(tr["v_cache"][ar, :, pos])
        kinb.copy_(tr["k_idx_cache"][ar, :, pos])
        lens.copy_(torch.tensor(hl, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        eo, es = msa.msa_decode_step_varlen(qb, qib, knb, vnb, kinb, ekc, evc, eos, ebk, hl, bs, k, return_sel=True)
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(sel, es), f"step {i}: the replay differs from the eager step"
    assert torch.equal(kc, ekc) and torch.equal(vc, evc) and torch.equal(bk, ebk) and torch.equal(osum, eos)
