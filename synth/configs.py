"""The five synthetic MSA workloads (shapes, block size, selection budget).

``top_k`` counts the query's own block: a query ranks ``top_k - 1`` earlier
blocks and always adds its own.
"""
from dataclasses import dataclass, asdict


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    batch: int
    seq_len: int         # S for prefill, cache length L for decode
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    idx_dim: int
    block_size: int
    top_k: int
    structured: bool = False   # hot-block index keys (non-uniform selection)
    hot_fraction: float = 0.05

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block_size)

    @property
    def group_size(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def as_dict(self):
        return asdict(self)


WORKLOADS = {
    "tiny_2k": Workload("tiny_2k", "prefill", 1, 2048, 8, 1, 128, 64, 64, 8),
    "prefill_32k": Workload("prefill_32k", "prefill", 1, 32768, 64, 8, 128, 64, 128, 16),
    "structured_128k": Workload("structured_128k", "prefill", 1, 131072, 64, 8, 128, 64, 128, 16,
                                structured=True),
    "decode_b16_256k": Workload("decode_b16_256k", "decode", 16, 262144, 64, 8, 128, 64, 128, 16),
    "prefill_1m": Workload("prefill_1m", "prefill", 1, 1048576, 64, 8, 128, 64, 128, 16),
}


def get_workload(name: str, **overrides) -> Workload:
    base = WORKLOADS[name]
    if not overrides:
        return base
    d = base.as_dict()
    d.update(overrides)
    return Workload(**d)
