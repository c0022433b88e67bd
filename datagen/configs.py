"""Workload shapes for the MoE FFN layer (the expert-node side of disaggregated
expert parallelism).

Notation follows the FinDEP review page ("FinDEP: Efficient MoE Inference with
Fine-Grained Scheduling of Disaggregated Expert Parallelism", section 核心公式 and
the input list of Algorithm 1): N tokens, hidden size M, E experts resident on
this GPU, top-k, expert (SwiGLU) width H, S shared experts of width Hs.

This module holds shapes only; it performs none of the layer's arithmetic.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str            # short key
    title: str           # what the workload is, with its sizes
    cfg_id: int          # seed namespace (SeedSequence entropy word 0)
    N: int               # tokens (rows for the pre-routed expert-node share)
    M: int               # hidden size
    E: int               # experts on this GPU
    k: int               # experts per token
    H: int               # expert SwiGLU width
    S: int = 0           # shared (always-on) experts
    Hs: int = 0          # width of each shared expert
    skewed_bias: bool = False   # per-expert router bias with Zipf-shaped popularity
    pre_routed: bool = False    # ids/weights are inputs (expert-node share), no router
    x_rows: int = 0      # rows generated for x (prefix reuse across an N sweep); 0 = N
    n_sweep: Tuple[int, ...] = field(default_factory=tuple)

    @property
    def A(self) -> int:
        """Assignments: k rows per token (the page on MoE latency, section
        "router 之后还有一串动作": top-2 gives 2N assignments)."""
        return self.N * self.k

    def with_tokens(self, n: int) -> "Workload":
        return replace(self, N=n)


TINY = Workload("tiny", "tiny MoE layer N=64 M=256 E=8 k=2 H=512", 1,
                N=64, M=256, E=8, k=2, H=512)
MIXTRAL = Workload("mixtral", "Mixtral-8x22B-shaped decode batch N=156 M=6144 E=8 k=2 H=16384", 2,
                   N=156, M=6144, E=8, k=2, H=16384)
DSV2 = Workload("dsv2", "DeepSeek-V2-shaped prefill N=4096 M=5120 E=160 k=6 H=1536 + 2x1536 shared", 3,
                N=4096, M=5120, E=160, k=6, H=1536, S=2, Hs=1536)
QWEN30 = Workload("qwen30", "Qwen3-30B-A3B-shaped decode M=2048 E=128 k=8 H=768", 4,
                  N=512, M=2048, E=128, k=8, H=768, x_rows=512, n_sweep=(1, 8, 32, 128, 512))
QWEN235 = Workload("qwen235", "Qwen3-235B-shaped skewed layer N=8192 M=4096 E=128 k=8 H=1536, Zipf(1.2) bias", 5,
                   N=8192, M=4096, E=128, k=8, H=1536, skewed_bias=True)
QWEN235_NODE = Workload("qwen235_node", "expert-node share: 16 local experts, 32768 pre-routed rows, M=4096 H=1536", 6,
                        N=32768, M=4096, E=16, k=1, H=1536, pre_routed=True)

ALL = {w.name: w for w in (TINY, MIXTRAL, DSV2, QWEN30, QWEN235, QWEN235_NODE)}


def get(name: str, n_tokens: Optional[int] = None) -> Workload:
    w = ALL[name]
    return w.with_tokens(n_tokens) if n_tokens is not None else w
