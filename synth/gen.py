"""Seeded generators for MSA inputs.

Layouts (the library's layouts):
  q        [B, S, Hq, D]   bf16      k, v       [B, Hkv, S, D] bf16
  q_idx    [B, G, S, di]   int8      k_idx      [B, G, S, di]  int8
  decode:  q [B, Hq, D] bf16, q_idx [B, G, di] int8,
           k_cache / v_cache [B, Hkv, L, D] bf16, k_idx_cache [B, G, L, di] int8

Distributions: bf16 tensors are N(0, 1) drawn in fp32 and rounded to bf16
(round-to-nearest-even, torch's conversion); int8 index tensors are uniform
on [-64, 63].  The structured workload plants hot blocks: per group a
direction u_g ~ U[-64, 63]^di, a seeded 5 % of blocks whose tokens' index
keys are clip(u_g + U[-8, 7]), and every query index vector is
clip(floor(u_g / 2) + U[-32, 31]), so queries prefer the hot blocks.

Every tensor is generated in fixed token chunks, each from its own seed
derived from (seed, tensor name, batch, chunk), so the values do not depend
on how much memory the device has.  torch's CPU and GPU generators differ, so
a run that feeds the oracle copies the device tensors to the host.
"""
import hashlib

import numpy as np
import torch

from .configs import Workload

CHUNK_TOKENS = 8192


def seed_for(*parts) -> int:
    """A stable 63-bit seed from any printable parts."""
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*parts))
    return g


def _normal_bf16(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def _uniform_i8(shape, gen, device, lo=-64, hi=64):
    return torch.randint(lo, hi, shape, generator=gen, device=device, dtype=torch.int8)


def _fill_token_major(out, name, seed, device, kind, tok_dim):
    """Fill ``out`` chunk by chunk along ``tok_dim`` (per batch entry)."""
    B = out.shape[0]
    S = out.shape[tok_dim]
    for b in range(B):
        for c0 in range(0, S, CHUNK_TOKENS):
            n = min(CHUNK_TOKENS, S - c0)
            view = out[b].narrow(tok_dim - 1, c0, n)
            g = _gen(device, seed, name, b, c0)
            if kind == "normal":
                view.copy_(_normal_bf16(tuple(view.shape), g, device))
            else:
                view.copy_(_uniform_i8(tuple(view.shape), g, device))


def prefill_inputs(w: Workload, seed: int = 0, device="cpu", seq_len=None, batch=None):
    """q, k, v, q_idx, k_idx for a prefill workload (optionally resized)."""
    B = batch if batch is not None else w.batch
    S = seq_len if seq_len is not None else w.seq_len
    Hq, G, D, di = w.n_q_heads, w.n_kv_heads, w.head_dim, w.idx_dim
    dev = torch.device(device)
    q = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((B, G, S, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty((B, G, S, D), dtype=torch.bfloat16, device=dev)
    q_idx = torch.empty((B, G, S, di), dtype=torch.int8, device=dev)
    k_idx = torch.empty((B, G, S, di), dtype=torch.int8, device=dev)
    _fill_token_major(q, "q", seed, dev, "normal", 1)
    _fill_token_major(k, "k", seed, dev, "normal", 2)
    _fill_token_major(v, "v", seed, dev, "normal", 2)
    _fill_token_major(q_idx, "q_idx", seed, dev, "int8", 2)
    _fill_token_major(k_idx, "k_idx", seed, dev, "int8", 2)
    if w.structured:
        _plant_hot_blocks(q_idx, k_idx, w, seed, dev)
    return {"q": q, "k": k, "v": v, "q_idx": q_idx, "k_idx": k_idx}


def grad_output(w: Workload, seed: int = 0, device="cpu", seq_len=None, batch=None):
    """dout [B, S, Hq, D] bf16 ~ N(0, 1): the gradient arriving at the
    attention output in a backward pass."""
    B = batch if batch is not None else w.batch
    S = seq_len if seq_len is not None else w.seq_len
    dev = torch.device(device)
    dout = torch.empty((B, S, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    _fill_token_major(dout, "dout", seed, dev, "normal", 1)
    return dout


def hot_blocks(w: Workload, seed: int, b: int, g: int, n_blocks: int):
    """Indices of the planted hot blocks of (b, g) (sorted)."""
    n_hot = max(1, int(round(w.hot_fraction * n_blocks)))
    perm = torch.randperm(n_blocks, generator=_gen("cpu", seed, "hot", b, g))
    return torch.sort(perm[:n_hot]).values


def _plant_hot_blocks(q_idx, k_idx, w, seed, dev):
    B, G, S, di = q_idx.shape
    bs = w.block_size
    nb = -(-S // bs)
    for b in range(B):
        for g in range(G):
            u = torch.randint(-64, 64, (di,), generator=_gen("cpu", seed, "dir", b, g),
                              dtype=torch.int32).to(dev)
            hot = hot_blocks(w, seed, b, g, nb).tolist()
            for j in hot:
                t0, t1 = j * bs, min(S, (j + 1) * bs)
                noise = torch.randint(-8, 8, (t1 - t0, di), generator=_gen("cpu", seed, "hotk", b, g, j),
                                      dtype=torch.int32).to(dev)
                k_idx[b, g, t0:t1] = torch.clamp(u[None, :] + noise, -128, 127).to(torch.int8)
            half = torch.div(u, 2, rounding_mode="floor")
            for c0 in range(0, S, CHUNK_TOKENS):
                n = min(CHUNK_TOKENS, S - c0)
                noise = torch.randint(-32, 32, (n, di), generator=_gen(dev, seed, "hotq", b, g, c0),
                                      device=dev, dtype=torch.int32)
                q_idx[b, g, c0:c0 + n] = torch.clamp(half[None, :] + noise, -128, 127).to(torch.int8)


def decode_inputs(w: Workload, seed: int = 0, device="cpu", seq_len=None, batch=None):
    """q, q_idx, k_cache, v_cache and per-token cache index keys for decode."""
    B = batch if batch is not None else w.batch
    L = seq_len if seq_len is not None else w.seq_len
    Hq, G, D, di = w.n_q_heads, w.n_kv_heads, w.head_dim, w.idx_dim
    dev = torch.device(device)
    q = _normal_bf16((B, Hq, D), _gen(dev, seed, "dq"), dev)
    q_idx = _uniform_i8((B, G, di), _gen(dev, seed, "dq_idx"), dev)
    k_cache = torch.empty((B, G, L, D), dtype=torch.bfloat16, device=dev)
    v_cache = torch.empty((B, G, L, D), dtype=torch.bfloat16, device=dev)
    k_idx_cache = torch.empty((B, G, L, di), dtype=torch.int8, device=dev)
    _fill_token_major(k_cache, "dk", seed, dev, "normal", 2)
    _fill_token_major(v_cache, "dv", seed, dev, "normal", 2)
    _fill_token_major(k_idx_cache, "dk_idx", seed, dev, "int8", 2)
    return {"q": q, "q_idx": q_idx, "k_cache": k_cache, "v_cache": v_cache,
            "k_idx_cache": k_idx_cache}


def sample_rows(S: int, n: int, seed: int = 0) -> np.ndarray:
    """``n`` distinct query positions in [0, S), sorted; all of them if n >= S."""
    if n >= S:
        return np.arange(S, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed_for(seed, "sample", S, n)))
    return np.sort(rng.choice(S, size=n, replace=False)).astype(np.int64)
