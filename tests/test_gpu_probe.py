"""The matrix-core probe (msa_probe_mfma_bf16), a measurement aid beside the
published bf16 peak: its output must be what the products it claims to run
give, so that its rate counts real MFMAs.

Every lane's A operand holds bf16 0x3a80 + (lane % 8) in the low and 0x3a80
in the high half of each word, B holds 0x3a81 in both; so row m of A is
(x_j, x_0, x_j, x_0, ...) over the 16 k with j = m % 8 (the lanes holding
row m share m % 8), and one product adds t_m = 8 (x_j + x_0) x_b to every
element of row m.  Each t_m has at most 16 significant bits, so 200 rounds
accumulate exactly in fp32; the thread's output is the sum, in order, of
its 4 x 16 accumulator elements (element i of lane l is row
8 (i / 4) + 4 (l / 32) + i % 4), replayed here in fp32."""
import numpy as np
import pytest
import torch

import block_sparse_attention_33_amd as msa

pytestmark = pytest.mark.gpu


def _bf16(bits):
    return np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]


def _expected(iters):
    x0, xb = _bf16(0x3A80), _bf16(0x3A81)
    out = np.zeros(256, dtype=np.float32)
    for tid in range(256):
        lane = tid & 63
        s = np.float32(0.0)
        for _c in range(4):
            for i in range(16):
                row = 8 * (i // 4) + 4 * (lane // 32) + i % 4
                t = np.float32(8.0) * (np.float32(_bf16(0x3A80 + (row & 7))) + x0) * xb
                s = np.float32(s + np.float32(iters) * t)
        out[tid] = s
    return out


def test_mfma_probe_output_and_flop():
    nwg, iters = 16, 200
    print(f"[probe] mfma probe {nwg} workgroups x {iters} rounds", flush=True)
    buf = torch.full((nwg * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    flop = msa.msa_probe_mfma_bf16(nwg, iters, buf)
    torch.cuda.synchronize()
    assert flop == nwg * 4 * iters * 4 * 2 * 32 * 32 * 16
    got = buf.cpu().numpy().reshape(nwg, 256)
    exp = _expected(iters)
    for w in range(nwg):
        np.testing.assert_array_equal(got[w], exp)
