"""Shared helpers of the GPU parity tests: host copies of device inputs for
the oracle and the output comparison."""
import numpy as np
import torch

from oracle import msa_oracle as O

MAX_ABS = 1e-2     # max |gpu - bf16(oracle)| over compared elements
MEAN_ABS = 1e-3    # mean |gpu - bf16(oracle)| over compared elements


def host_f32(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> float32 numpy (exact)."""
    return t.detach().to("cpu").float().numpy()


class HostBf16:
    """A host copy of a bf16 tensor that hands out float32 numpy slices, so
    the oracle can gather rows of a large cache without a full fp32 copy."""

    def __init__(self, t: torch.Tensor):
        self.t = t.detach().to("cpu")
        self.shape = tuple(self.t.shape)

    def __getitem__(self, idx):
        idx = tuple(torch.as_tensor(i) if isinstance(i, np.ndarray) else i for i in idx) \
            if isinstance(idx, tuple) else idx
        return self.t[idx].float().numpy()


def host_i8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").numpy()


def compare_out(gpu_bf16: torch.Tensor, oracle_f64: np.ndarray, what: str):
    """Compare a GPU bf16 output with the oracle rounded to bf16."""
    g = host_f32(gpu_bf16).astype(np.float64)
    ref = O.round_to_bf16(oracle_f64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    d = np.abs(g - ref)
    max_abs, mean_abs = float(d.max()), float(d.mean())
    assert max_abs <= MAX_ABS and mean_abs <= MEAN_ABS, (
        f"{what}: max_abs={max_abs:.3e} (<= {MAX_ABS}), mean_abs={mean_abs:.3e} (<= {MEAN_ABS}), "
        f"worst at {np.unravel_index(int(d.argmax()), d.shape)}")
    return max_abs, mean_abs


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
