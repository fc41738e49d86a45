"""The five decode workloads, as named presets.

Shapes follow the problem statement of this build (tiny c4a, 64K c128a, 128K
c4a with indexer, mixed paged batch, 1M 61-layer stack) and the pages' model
description ([V4-vLLM] 2.1: 61 layers, the first 30 c4a and the last 31 c128a,
a c4a entry folding an 8-token window at stride 4; 2.3: a 128-token window;
3.1.1: 256-token logical blocks).
"""

from dataclasses import dataclass, field
from typing import List, Optional


@dataclass(frozen=True)
class LayerKind:
    name: str  # "c4a" | "c128a"
    m: int
    topk: Optional[int]  # None: all entries attended
    idx_dtype: Optional[str] = None  # indexer key storage for c4a
    d_idx: int = 0
    h_idx: int = 16
    overlap: int = 0  # tokens of the previous group in each entry's window (c4a: 4, an 8-token window)

    @property
    def slots(self) -> int:
        """Slots of a compressor window (the length of its slot biases)."""
        return self.m + self.overlap


@dataclass
class Workload:
    cid: int
    name: str
    B: int
    L: Optional[int]  # fixed context length, or None for drawn lengths
    d: int
    H: int
    window: int
    kv_dtype: str
    layers: List[LayerKind]
    table: str = "perm"  # "identity" | "perm"
    L_range: Optional[tuple] = None  # (lo, hi) for log-uniform lengths
    shared_prefix_seqs: int = 0
    shared_prefix_blocks: int = 0
    theta: float = 1.0e6
    token_std: float = 1.0
    beta_std: float = 0.1
    extra: dict = field(default_factory=dict)


C4A_TINY = LayerKind("c4a", 4, 256, "bf16", 64, 16, overlap=4)
C4A_FP8 = LayerKind("c4a", 4, 2048, "fp8", 128, 16, overlap=4)
C4A_FP4 = LayerKind("c4a", 4, 2048, "fp4", 128, 16, overlap=4)
C128A = LayerKind("c128a", 128, None)

CONFIGS = {
    0: Workload(0, "tiny-c4a-4k", 1, 4096, 128, 8, 128, "bf16", [C4A_TINY], table="identity"),
    1: Workload(1, "c128a-64k-b8", 8, 65536, 512, 64, 128, "fp8", [C128A]),
    2: Workload(2, "c4a-128k-b16-topk2048", 16, 131072, 512, 64, 128, "fp8", [C4A_FP8]),
    3: Workload(3, "mixed-paged-b64", 64, None, 512, 64, 128, "fp8", [C4A_FP8, C128A],
                L_range=(256, 131072), shared_prefix_seqs=16, shared_prefix_blocks=8),
    4: Workload(4, "stack-1m-b4-61layers", 4, 1 << 20, 512, 64, 128, "fp8",
                [C4A_FP4] * 30 + [C128A] * 31),
}


def workload(cid: int) -> Workload:
    return CONFIGS[cid]
