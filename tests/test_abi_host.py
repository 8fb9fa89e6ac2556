"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/msa.h declares, rejects bad arguments with the
documented status before touching the GPU, and sizes workspaces by the
documented layout."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_33_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_33_amd import build
        build.build()
    return _lib.load()


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["msa_index_select", "msa_prefill", "msa_decode", "msa_workspace_bytes",
              "msa_pool_block_keys", "msa_status_string", "msa_version", "msa_decode_init",
              "msa_decode_step", "msa_prefill_chunk", "msa_prefill_chunk_workspace_bytes", "msa_prefill_lse",
              "msa_prefill_backward"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(_lib.SIGNATURES), "binding signatures out of sync with msa.h"


def test_status_strings(lib):
    for code, prefix in [(0, "MSA_OK"), (-1, "MSA_ERR_INVALID_ARG"), (-2, "MSA_ERR_UNSUPPORTED"),
                         (-3, "MSA_ERR_WORKSPACE"), (-4, "MSA_ERR_HIP"), (-5, "MSA_ERR_SCRATCH")]:
        assert lib.msa_status_string(code).decode().startswith(prefix)
    assert lib.msa_status_string(12345).decode() == "unknown MSA status"
    assert lib.msa_version() == 10900


def D(**kw):
    base = dict(batch=1, seq_len=4096, n_q_heads=64, n_kv_heads=8, head_dim=128, idx_dim=64,
                block_size=128, top_k=16, softmax_scale=0.0)
    base.update(kw)
    return _lib.MsaDims(**base)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _ws(lib, op, dims):
    lo, hi = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib.msa_workspace_bytes(op, ctypes.byref(dims), ctypes.byref(lo), ctypes.byref(hi))
    return st, lo.value, hi.value


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -1), (dict(seq_len=-5), -1), (dict(n_q_heads=63), -1), (dict(top_k=0), -1),
    (dict(softmax_scale=float("nan")), -1), (dict(softmax_scale=float("inf")), -1),
    (dict(head_dim=64), -2), (dict(idx_dim=32), -2), (dict(block_size=96), -2),
    (dict(block_size=256), -2), (dict(top_k=33, seq_len=8192), -2), (dict(n_q_heads=24), -2),
    (dict(n_q_heads=256), -2), (dict(seq_len=1 << 26), -2),
    (dict(batch=64, seq_len=1 << 20), -2),
])
def test_dims_validation(lib, kw, code):
    dims = D(**kw)
    st, _, _ = _ws(lib, _lib.MSA_OP_PREFILL, dims)
    assert st == code
    out = lib.msa_prefill(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert out == code


def test_dense_top_k(lib):
    """top_k >= nb: a dense prefill with no workspace, any top_k; the sparse
    entry points still keep at most 32 blocks."""
    dims = D(seq_len=8192, top_k=64)  # nb = 64
    assert _ws(lib, _lib.MSA_OP_PREFILL, dims) == (0, 0, 0)
    for op in (_lib.MSA_OP_INDEX, _lib.MSA_OP_DECODE):
        assert _ws(lib, op, dims)[0] == -2
    assert lib.msa_decode(ctypes.byref(dims), *([FAKE] * 6), None, FAKE, 1 << 30, None) == -2
    assert lib.msa_prefill_chunk(ctypes.byref(dims), 0, 10, *([FAKE] * 7), None, FAKE, 1 << 30, None) == -2
    assert _ws(lib, _lib.MSA_OP_PREFILL, D(seq_len=4096, top_k=16))[1] > 0  # nb = 32 > 16: sparse


def test_null_pointers(lib):
    dims = D()
    assert lib.msa_prefill(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == -1
    for i in range(6):
        args = [FAKE] * 6
        args[i] = None
        assert lib.msa_prefill(ctypes.byref(dims), *args, None, FAKE, 1 << 40, None) == -1
    assert lib.msa_index_select(ctypes.byref(dims), FAKE, FAKE, FAKE, None, None, 0, None) == -1
    assert lib.msa_pool_block_keys(ctypes.byref(dims), None, FAKE, None) == -1
    for i in range(6):
        args = [FAKE] * 6
        args[i] = None
        assert lib.msa_decode(ctypes.byref(dims), *args, None, FAKE, 1 << 40, None) == -1


def test_decode_step_validation(lib):
    """The generation calls reject bad lengths and null pointers before any
    launch (dims.seq_len is the cache capacity)."""
    dims = D(batch=2, seq_len=1000)
    st, lo, _ = _ws(lib, _lib.MSA_OP_DECODE, dims)
    assert st == 0
    for length in (0, -1, 1001):
        assert lib.msa_decode_step(ctypes.byref(dims), length, *([FAKE] * 10), None, FAKE, lo, None) == -1
    for i in range(10):
        args = [FAKE] * 10
        args[i] = None
        assert lib.msa_decode_step(ctypes.byref(dims), 10, *args, None, FAKE, lo, None) == -1
    assert lib.msa_decode_step(ctypes.byref(dims), 10, *([FAKE] * 10), None, FAKE, lo - 1, None) == -3
    assert lib.msa_decode_step(ctypes.byref(D(head_dim=64)), 10, *([FAKE] * 10), None, FAKE, lo, None) == -2
    for length in (-1, 1001):
        assert lib.msa_decode_init(ctypes.byref(dims), length, FAKE, FAKE, FAKE, None) == -1
    for i in range(3):
        args = [FAKE] * 3
        args[i] = None
        assert lib.msa_decode_init(ctypes.byref(dims), 10, *args, None) == -1
    assert lib.msa_decode_init(ctypes.byref(dims), 0, FAKE, FAKE, FAKE, None) == 0  # nothing to enqueue


def test_prefill_chunk_validation(lib):
    """Chunked prefill: start/count must lie inside the capacity; null
    pointers and short workspaces are rejected before any launch."""
    dims = D(batch=1, seq_len=4096)
    lo, hi = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.msa_prefill_chunk_workspace_bytes(ctypes.byref(dims), 1024, ctypes.byref(lo), ctypes.byref(hi)) == 0
    assert 0 < lo.value <= hi.value
    for count in (0, -3, 4097):
        assert lib.msa_prefill_chunk_workspace_bytes(ctypes.byref(dims), count, None, None) == -1
    # the workspace of a chunk grows with the chunk, not with the capacity's tokens
    lo2 = ctypes.c_size_t(0)
    assert lib.msa_prefill_chunk_workspace_bytes(ctypes.byref(dims), 2048, ctypes.byref(lo2), None) == 0
    assert lo2.value > lo.value
    for start, count in ((-1, 10), (0, 0), (4000, 97), (4096, 1)):
        assert lib.msa_prefill_chunk(ctypes.byref(dims), start, count, *([FAKE] * 7), None, FAKE, hi.value,
                                     None) == -1
    for i in range(7):
        args = [FAKE] * 7
        args[i] = None
        assert lib.msa_prefill_chunk(ctypes.byref(dims), 0, 1024, *args, None, FAKE, hi.value, None) == -1
    assert lib.msa_prefill_chunk(ctypes.byref(dims), 0, 1024, *([FAKE] * 7), None, FAKE, lo.value - 1,
                                 None) == -3


def test_prefill_chunk_varlen_validation(lib):
    """Ragged chunked prefill: every sequence's start and count must lie
    inside the capacity (a count of 0 skips the sequence, but some sequence
    must add a query); null pointers are refused; every sequence's plan is
    checked against the workspace -- the largest chunk's, for a batch of
    one -- before any launch."""
    dims = D(batch=3, seq_len=4096, n_q_heads=8, n_kv_heads=2)
    args = [FAKE] * 7  # q, q_idx, k_cache, v_cache, k_idx, block_keys, out
    one = D(batch=1, seq_len=4096, n_q_heads=8, n_kv_heads=2)
    lo = ctypes.c_size_t(0)
    assert lib.msa_prefill_chunk_workspace_bytes(ctypes.byref(one), 2000, ctypes.byref(lo), None) == 0
    starts, counts = _cu(0, 100, 4000), _cu(2000, 0, 96)
    for bad_s, bad_c in (((-1, 100, 4000), (2000, 0, 96)), ((0, 100, 4001), (2000, 0, 96)),
                         ((0, 100, 4000), (2000, -1, 96)), ((0, 100, 4000), (4097, 0, 96)),
                         ((0, 0, 0), (0, 0, 0))):
        assert lib.msa_prefill_chunk_varlen(ctypes.byref(dims), _cu(*bad_s), _cu(*bad_c), *args, None, FAKE,
                                            1 << 40, None) == -1
    assert lib.msa_prefill_chunk_varlen(ctypes.byref(dims), None, counts, *args, None, FAKE, 1 << 40, None) == -1
    assert lib.msa_prefill_chunk_varlen(ctypes.byref(dims), starts, None, *args, None, FAKE, 1 << 40, None) == -1
    for i in range(7):
        a = list(args)
        a[i] = None
        assert lib.msa_prefill_chunk_varlen(ctypes.byref(dims), starts, counts, *a, None, FAKE, 1 << 40,
                                            None) == -1
    # below the largest chunk's minimum, or no workspace: refused before anything is enqueued
    assert lib.msa_prefill_chunk_varlen(ctypes.byref(dims), starts, counts, *args, None, FAKE, lo.value - 256,
                                        None) == -3
    assert lib.msa_prefill_chunk_varlen(ctypes.byref(dims), starts, counts, *args, None, None, 1 << 40,
                                        None) == -3
    assert lib.msa_prefill_chunk_varlen(ctypes.byref(D(batch=3, seq_len=4096, n_q_heads=8, n_kv_heads=2,
                                                       top_k=40)), starts, counts, *args, None, FAKE, 1 << 40,
                                        None) == -2


def test_decode_varlen_validation(lib):
    """Ragged decode, init and step: the host lengths must lie in 1 .. C
    (0 .. C for init); null pointers and short workspaces are refused before
    any launch; the workspace is msa_decode's."""
    dims = D(batch=3, seq_len=5000, n_q_heads=8, n_kv_heads=2)
    st, lo, hi = _ws(lib, _lib.MSA_OP_DECODE, dims)
    assert st == 0 and lo > 0
    good = _cu(1, 4999, 5000)
    args = [FAKE] * 6  # q, q_idx, k_cache, v_cache, block_keys, out
    for bad in (None, _cu(0, 10, 20), _cu(1, 5001, 20), _cu(-1, 10, 20)):
        assert lib.msa_decode_varlen(ctypes.byref(dims), bad, *args, None, FAKE, hi, None) == -1
        assert lib.msa_decode_step_varlen(ctypes.byref(dims), bad, *([FAKE] * 10), None, FAKE, hi, None) == -1
    for i in range(6):
        a = list(args)
        a[i] = None
        assert lib.msa_decode_varlen(ctypes.byref(dims), good, *a, None, FAKE, hi, None) == -1
    for i in range(10):
        a = [FAKE] * 10
        a[i] = None
        assert lib.msa_decode_step_varlen(ctypes.byref(dims), good, *a, None, FAKE, hi, None) == -1
    assert lib.msa_decode_varlen(ctypes.byref(dims), good, *args, None, FAKE, lo - 1, None) == -3
    assert lib.msa_decode_varlen(ctypes.byref(dims), good, *args, None, None, hi, None) == -3
    assert lib.msa_decode_step_varlen(ctypes.byref(dims), good, *([FAKE] * 10), None, FAKE, lo - 1, None) == -3
    for bad in (None, _cu(0, 10, 5001), _cu(-1, 0, 0)):
        assert lib.msa_decode_init_varlen(ctypes.byref(dims), bad, FAKE, FAKE, FAKE, None) == -1
    assert lib.msa_decode_init_varlen(ctypes.byref(dims), _cu(0, 0, 0), None, FAKE, FAKE, None) == -1
    # all lengths 0: nothing to pool, nothing enqueued
    assert lib.msa_decode_init_varlen(ctypes.byref(dims), _cu(0, 0, 0), FAKE, FAKE, FAKE, None) == 0


def test_decode_varlen_device_validation(lib):
    """Device-resident lengths: the pointers (lengths included) must be
    given and the workspace must hold msa_decode's; the values themselves
    are checked by the kernels, not here."""
    dims = D(batch=3, seq_len=5000, n_q_heads=8, n_kv_heads=2)
    st, lo, hi = _ws(lib, _lib.MSA_OP_DECODE, dims)
    for i in range(7):  # lengths, q, q_idx, k_cache, v_cache, block_keys, out
        a = [FAKE] * 7
        a[i] = None
        assert lib.msa_decode_varlen_device(ctypes.byref(dims), *a, None, FAKE, hi, None) == -1
    for i in range(11):
        a = [FAKE] * 11
        a[i] = None
        assert lib.msa_decode_step_varlen_device(ctypes.byref(dims), *a, None, FAKE, hi, None) == -1
    assert lib.msa_decode_varlen_device(ctypes.byref(dims), *([FAKE] * 7), None, FAKE, lo - 1, None) == -3
    assert lib.msa_decode_step_varlen_device(ctypes.byref(dims), *([FAKE] * 11), None, None, hi, None) == -3
    big_k = D(batch=3, seq_len=5000, n_q_heads=8, n_kv_heads=2, top_k=40)
    assert lib.msa_decode_varlen_device(ctypes.byref(big_k), *([FAKE] * 7), None, FAKE, 1 << 30, None) == -2


def test_mfma_probe_validation(lib):
    """The matrix-core probe checks its arguments before any launch: 1 ..
    2^20 workgroups, 1 .. 2^24 rounds, an output buffer."""
    flop = ctypes.c_double(-1.0)
    for nw, it, out in [(0, 10, FAKE), ((1 << 20) + 1, 10, FAKE), (8, 0, FAKE), (8, (1 << 24) + 1, FAKE),
                        (8, 10, None)]:
        assert lib.msa_probe_mfma_bf16(nw, it, out, ctypes.byref(flop), None) == -1
    assert flop.value == -1.0  # nothing reported for a rejected call


def test_backward_validation(lib):
    """Training path: msa_prefill_lse needs its lse output; the backward
    needs every tensor, a workspace of its documented size (one bf16 dq
    partial per (query row, kept block) and head), and top_k <= 32."""
    dims = D(batch=2, seq_len=3000, top_k=8)
    for i in range(7):
        args = [FAKE] * 7
        args[i] = None
        assert lib.msa_prefill_lse(ctypes.byref(dims), *args[:6], None, args[6], FAKE, 1 << 40, None) == -1
    st, lo, hi = _ws(lib, _lib.MSA_OP_BACKWARD, dims)
    assert st == 0 and lo < hi
    part = 2 * 64 * 3000 * 8 * 128 * 2          # B * Hq * S * top_k * D * bf16
    assert part < hi < part + 2 * 3000 * 64 * 4 + 40 * 2 * 8 * 3000 * 8 + (1 << 20)
    # the least workspace runs passes of 256 query rows and keeps fp32 sums of
    # dK and dV (2 * B * G * S * D * 4 bytes)
    acc = 2 * 2 * 8 * 3000 * 128 * 4
    part256 = 2 * 64 * 256 * 8 * 128 * 2
    assert acc + part256 < lo < acc + part256 + 2 * 3000 * 64 * 4 + (4 << 20)
    # pass planning on the host: full -> one pass, least -> 256 rows, in
    # between a multiple of 256 that grows with the workspace, below -> 0
    rows = ctypes.c_int32(-1)
    for size, want in ((hi, 3000), (lo, 256), (lo - 1, 0), (0, 0)):
        assert lib.msa_backward_pass_rows(ctypes.byref(dims), size, ctypes.byref(rows)) == 0
        assert rows.value == want, (size, rows.value, want)
    prev = 256
    for f in (0.2, 0.5, 0.9):
        assert lib.msa_backward_pass_rows(ctypes.byref(dims), lo + int((hi - lo) * f), ctypes.byref(rows)) == 0
        assert rows.value % 256 == 0 and prev <= rows.value < 3000, (f, rows.value)
        prev = rows.value
    assert lib.msa_backward_pass_rows(ctypes.byref(dims), hi, None) == -1
    # a sequence of at most 256 rows runs in one pass: min = full
    st, lo1, hi1 = _ws(lib, _lib.MSA_OP_BACKWARD, D(batch=1, seq_len=256, top_k=2))
    assert st == 0 and lo1 == hi1
    for i in range(10):
        args = [FAKE] * 10
        args[i] = None
        assert lib.msa_prefill_backward(ctypes.byref(dims), *args, FAKE, lo, None) == -1
    assert lib.msa_prefill_backward(ctypes.byref(dims), *([FAKE] * 10), FAKE, lo - 1, None) == -3
    assert lib.msa_prefill_backward(ctypes.byref(dims), *([FAKE] * 10), ctypes.c_void_p(0x1008), lo, None) == -3
    assert lib.msa_prefill_backward(ctypes.byref(dims), *([FAKE] * 10), None, 0, None) == -3
    big_k = D(seq_len=4096, top_k=64)            # dense forward, but no sparse backward
    assert _ws(lib, _lib.MSA_OP_BACKWARD, big_k)[0] == -2
    assert lib.msa_prefill_backward(ctypes.byref(big_k), *([FAKE] * 10), FAKE, 1 << 40, None) == -2


def test_workspace_errors(lib):
    dims = D()
    st, lo, hi = _ws(lib, _lib.MSA_OP_PREFILL, dims)
    assert st == 0 and 0 < lo <= hi
    assert lib.msa_prefill(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, lo, None) == -3
    assert lib.msa_prefill(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, lo - 1,
                           None) == -3
    misaligned = ctypes.c_void_p(0x1000 + 64)
    assert lib.msa_prefill(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, misaligned, hi,
                           None) == -3
    st, dlo, dhi = _ws(lib, _lib.MSA_OP_DECODE, dims)
    assert st == 0 and dlo == dhi > 0
    assert lib.msa_decode(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, dlo - 1,
                          None) == -3
    assert lib.msa_workspace_bytes(99, ctypes.byref(dims), None, None) == -1


def _a(x):
    return (x + 255) // 256 * 256


def _query_chunk(S):
    """Tokens per query chunk of a prefill: the whole sequence up to 16384,
    16384 up to 131072, a quarter of the sequence (a multiple of 16384)
    beyond."""
    if S <= 16384:
        return S
    if S <= 131072:
        return 16384
    return -(-(-(-S // 4)) // 16384) * 16384


def _plan(U, S, nb):
    """The documented prefill plan: one query range per unit, histogram
    chunks of a multiple of 256 tokens, at most 2^22 counters."""
    T = -(-S // 256) * 256
    m = max(1, min(T // 256, max(1, (1 << 22) // (U * nb))))
    tpc = -(-(T // 256) // m) * 256
    m = -(-T // tpc)
    return m


@pytest.mark.parametrize("B,S,Hq,G,bs,k", [
    (1, 32768, 64, 8, 128, 16), (1, 2048, 8, 1, 64, 8), (2, 1000, 8, 2, 32, 5),
    (1, 777, 16, 1, 128, 1), (1, 1048576, 64, 8, 128, 16), (1, 131072, 64, 8, 128, 16),
    (1, 65536, 8, 1, 128, 1), (1, 200000, 8, 1, 128, 4)])
def test_prefill_workspace_layout(lib, B, S, Hq, G, bs, k):
    """The documented layout: fixed part + one bf16 partial (r x 128) and one
    fp32 (max, sum) pair (r) per (token, kept block) of a pass; the
    token-sized parts cover one query chunk, the block-sized parts the whole
    sequence."""
    dims = D(batch=B, seq_len=S, n_q_heads=Hq, n_kv_heads=G, block_size=bs, top_k=k)
    st, lo, hi = _ws(lib, _lib.MSA_OP_PREFILL, dims)
    assert st == 0
    U, r = B * G, Hq // G
    nb = -(-S // bs)
    S = _query_chunk(S)
    tpi = 6 * 256 // r          # up to 6 chunks of 256 query rows per work item
    n_chunks = _plan(U, S, nb)
    rows = U * nb
    items = U * ((S * k + tpi - 1) // tpi + nb) + 1
    fixed = (_a(U * nb * 64) + _a(U * S * k * 4) + _a(rows * 4) + _a(U * n_chunks * nb * 4)
             + 2 * _a((rows + 1) * 4) + _a(U * S * k * 4) + _a(items * 8) + _a(4))
    part = lambda n: _a(n * S * k * r * 128 * 2) + _a(n * S * k * r * 8)  # noqa: E731
    assert lo == fixed + part(1)
    assert hi == fixed + part(U)


def test_prefill_block_limit(lib):
    assert _ws(lib, _lib.MSA_OP_PREFILL, D(seq_len=36864 * 32, block_size=32, top_k=2, n_kv_heads=1,
                                           n_q_heads=1))[0] == 0
    assert _ws(lib, _lib.MSA_OP_PREFILL, D(seq_len=36864 * 32 + 1, block_size=32, top_k=2, n_kv_heads=1,
                                           n_q_heads=1))[0] == -2


def test_decode_workspace_layout(lib):
    dims = D(batch=16, seq_len=262144)
    st, lo, hi = _ws(lib, _lib.MSA_OP_DECODE, dims)
    U, k, r = 16 * 8, 16, 8
    # the selection (when the caller passes no sel), two workgroup states
    # per unit: r x (128 + 2) fp32, and a ragged batch's lengths (int32 per
    # sequence)
    exp = _a(U * k * 4) + _a(U * 2 * r * 130 * 4) + _a(16 * 4)
    assert st == 0 and lo == hi == exp
    # at most 8192 candidate blocks before the own block
    assert _ws(lib, _lib.MSA_OP_DECODE, D(batch=1, seq_len=8193 * 128))[0] == 0
    assert _ws(lib, _lib.MSA_OP_DECODE, D(batch=1, seq_len=8193 * 128 + 1))[0] == -2
    assert _ws(lib, _lib.MSA_OP_INDEX, dims)[1:] == (0, 0)


def test_decode_noalloc_validation(lib):
    """The allocation-free decode rejects null pointers and shapes whose
    scratch exceeds the library's fixed array before anything is enqueued."""
    dims = D(batch=16, seq_len=262144)
    for i in range(6):
        args = [FAKE] * 6
        args[i] = None
        assert lib.msa_decode_noalloc(ctypes.byref(dims), *args, None, None) == -1
    # the decode workload's scratch fits; that of 524288 units (65536
    # sequences x 8 groups) does not
    st, lo, _ = _ws(lib, _lib.MSA_OP_DECODE, dims)
    assert st == 0 and lo <= _lib.MSA_DECODE_SCRATCH_BYTES
    big = D(batch=65536, seq_len=1)
    st, lo, _ = _ws(lib, _lib.MSA_OP_DECODE, big)
    assert st == 0 and lo > _lib.MSA_DECODE_SCRATCH_BYTES
    assert lib.msa_decode_noalloc(ctypes.byref(big), *([FAKE] * 6), None, None) == _lib.MSA_ERR_SCRATCH
    assert lib.msa_decode_noalloc(ctypes.byref(D(top_k=33)), *([FAKE] * 6), None, None) == -2


def _plan_check(lib, op, dims, ws):
    n = ctypes.c_int32(-1)
    st = lib.msa_plan_check(op, ctypes.byref(dims), ctypes.c_size_t(int(ws)), ctypes.byref(n))
    return st, n.value


def _rows_per_pass(lib, dims, ws):
    r = ctypes.c_int32(-1)
    assert lib.msa_backward_pass_rows(ctypes.byref(dims), ctypes.c_size_t(int(ws)), ctypes.byref(r)) == 0
    return r.value


# up to the longest supported prefill: 36864 blocks of 128 tokens
SWEEP_S = [1, 255, 256, 257, 4097, 32768, 300000, 1 << 20, 36864 * 128 - 5, 36864 * 128]


@pytest.mark.parametrize("S", SWEEP_S)
def test_plan_sweep_backward(lib, S):
    """For every sequence length above and a spread of workspaces between the
    backward's minimum and full size, every pass the call would run (the
    shorter last one included) plans its inversion inside the regions sized
    for the pass length; below the minimum the call is refused."""
    dims = D(seq_len=S)
    st, lo, hi = _ws(lib, _lib.MSA_OP_BACKWARD, dims)
    assert st == 0 and 0 < lo <= hi
    sizes = sorted({lo, hi, (lo + hi) // 2, lo + (hi - lo) // 7, lo + (hi - lo) // 64, lo + 12345,
                    max(lo, hi - 1)} | {int(lo + (hi - lo) * f) for f in (0.01, 0.03, 0.1, 0.27, 0.5, 0.9)})
    for ws in sizes:
        st, passes = _plan_check(lib, _lib.MSA_OP_BACKWARD, dims, ws)
        assert st == 0, (S, ws, st)
        rows = _rows_per_pass(lib, dims, ws)
        assert rows == S or (rows > 0 and rows % 256 == 0), (S, ws, rows)
        assert passes == -(-S // rows), (S, ws, rows, passes)
    if lo > 1:
        assert _plan_check(lib, _lib.MSA_OP_BACKWARD, dims, lo - 1)[0] == -3


@pytest.mark.parametrize("S", SWEEP_S)
def test_plan_sweep_prefill(lib, S):
    """Every query chunk of a prefill (the last, shorter one included) and
    every unit pass fits the workspace, for workspaces from the minimum to the
    full size; the summaries shared by the chunks sit at offset 0."""
    dims = D(seq_len=S)
    st, lo, hi = _ws(lib, _lib.MSA_OP_PREFILL, dims)
    assert st == 0
    if hi == 0:  # top_k >= nb: dense kernel, nothing planned
        assert _plan_check(lib, _lib.MSA_OP_PREFILL, dims, 0) == (0, 1)
        return
    for ws in sorted({lo, hi, (lo + hi) // 2, lo + (hi - lo) // 5, lo + 1000, max(lo, hi - 1)}):
        st, launches = _plan_check(lib, _lib.MSA_OP_PREFILL, dims, ws)
        assert st == 0 and launches >= 1, (S, ws, st)
    assert _plan_check(lib, _lib.MSA_OP_PREFILL, dims, hi)[1] == -(-S // max(1, min(S, _chunk_tokens(S))))
    assert _plan_check(lib, _lib.MSA_OP_PREFILL, dims, lo - 1)[0] == -3


def _chunk_tokens(S):
    """Query tokens per chunk of a whole prefill, as the library documents it:
    16384 up to 128K tokens, a quarter of the sequence (in whole 16384s) beyond."""
    if S <= 16384:
        return S
    if S <= 131072:
        return 16384
    quarter = -(-S // 4)
    return -(-quarter // 16384) * 16384


def test_plan_check_arguments(lib):
    # beyond 36864 blocks (here 2^26 - 1 tokens) neither call is supported
    for op in (_lib.MSA_OP_PREFILL, _lib.MSA_OP_BACKWARD):
        assert _plan_check(lib, op, D(seq_len=(1 << 26) - 1), 1 << 40)[0] == -2
        assert _plan_check(lib, op, D(seq_len=36864 * 128 + 1), 1 << 40)[0] == -2
    assert _plan_check(lib, 99, D(), 1 << 30)[0] == -1
    assert _plan_check(lib, _lib.MSA_OP_PREFILL, D(head_dim=64), 1 << 30)[0] == -2
    assert _plan_check(lib, _lib.MSA_OP_BACKWARD, D(), 0)[0] == -3


def _cu(*xs):
    return (ctypes.c_int32 * len(xs))(*xs)


def test_prefill_varlen_validation(lib):
    """Ragged-batch prefill: the host offsets are checked (start at 0,
    non-decreasing, no sequence longer than dims.seq_len, at least one token)
    and every sequence's plan is checked against the workspace before any
    launch; its workspace is the longest sequence's alone."""
    dims = D(batch=3, seq_len=5000, n_q_heads=8, n_kv_heads=2)
    args = [FAKE] * 7  # q, k, v, q_idx, k_idx, out, sel
    good = _cu(0, 100, 5100, 6000)
    for bad in (None, _cu(1, 100, 5100, 6000), _cu(0, 100, 50, 6000), _cu(0, 100, 5101, 6000), _cu(0, 0, 0, 0)):
        assert lib.msa_prefill_varlen(ctypes.byref(dims), bad, *args, FAKE, 1 << 40, None) == -1
    for i in range(6):
        a = list(args)
        a[i] = None
        assert lib.msa_prefill_varlen(ctypes.byref(dims), good, *a, FAKE, 1 << 40, None) == -1
    st, lo, hi = _ws(lib, _lib.MSA_OP_PREFILL_VARLEN, dims)
    one = D(batch=1, seq_len=5000, n_q_heads=8, n_kv_heads=2)
    assert st == 0 and (lo, hi) == _ws(lib, _lib.MSA_OP_PREFILL, one)[1:]
    assert lo > 0
    # below the longest sequence's minimum: refused before anything is enqueued
    assert lib.msa_prefill_varlen(ctypes.byref(dims), good, *args, FAKE, lo - 256, None) == -3
    assert lib.msa_prefill_varlen(ctypes.byref(dims), good, *args, None, 1 << 40, None) == -3


def test_prefill_switched_validation(lib):
    """The short-sequence switch: null pointers and unsupported shapes are
    refused before any launch on both routes; at or above the threshold the
    call is msa_prefill (top_k 33 < nb is unsupported there), below it any
    top_k >= 1 is accepted (standard attention does not use it)."""
    took = ctypes.c_int32(-7)
    assert lib.msa_prefill_switched(None, 0, *([FAKE] * 7), FAKE, 1 << 40, None, ctypes.byref(took)) == -1
    long_ = D(seq_len=20000, top_k=33)
    assert lib.msa_prefill_switched(ctypes.byref(long_), 0, *([FAKE] * 7), FAKE, 1 << 40, None,
                                    ctypes.byref(took)) == -2
    short = D(seq_len=4000, top_k=0)
    assert lib.msa_prefill_switched(ctypes.byref(short), 0, *([FAKE] * 7), FAKE, 1 << 40, None,
                                    ctypes.byref(took)) == -1
    short = D(seq_len=4000, top_k=16)
    a = [FAKE] * 7
    a[0] = None
    assert lib.msa_prefill_switched(ctypes.byref(short), 0, *a, None, 0, None, ctypes.byref(took)) == -1
    assert lib.msa_prefill_switched(ctypes.byref(D(seq_len=4000, head_dim=64)), 0, *([FAKE] * 7), None, 0, None,
                                    ctypes.byref(took)) == -2
