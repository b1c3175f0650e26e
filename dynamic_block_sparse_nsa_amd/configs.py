"""Workload configurations for the NSA forward pass.

Field names mirror the C struct ``nsa_config`` in ``include/nsa.h``.  The five named
workloads are the ones this library is measured and parity-checked on:

* ``tiny``   - batch 1, 1024 tokens, 1 KV head shared by a group of 4 query heads,
               d_k = d_v = 64, compression blocks of 32 with stride 16, 64-token
               selection blocks, top-4 (block 0 and the two local blocks forced),
               window 128.
* ``8k``     - batch 1, 8192 tokens, 4 KV groups x 16 query heads, d_k 192, d_v 128,
               compression 32/16, selection 64-token blocks, top-16 (1 initial + 2
               local forced), window 512.
* ``64k``    - the same architecture at 65536 tokens (the headline prefill shape).
* ``decode`` - batch 32, one new query per sequence against a 65536-token cache,
               same architecture as ``8k``.
* ``moba``   - MoBA-style mode: 131072 tokens, 8 query heads each with its own KV
               head, d 128, 512-token blocks keyed by mean-pooled K, per-head top-3
               with the current block forced; no compressed or window branch.

Sources: the three-branch NSA structure, GQA-shared selection, the 64-token/top-16 NSA
geometry and the 512-token/top-3 MoBA geometry are described on the zjai.club episode
notes (sections 5-8, 16-17 and the summary bullets); the d_k 192 / 4 groups x 16
heads shape is the one quoted there in section 8.
"""
from __future__ import annotations

import dataclasses
import math

PHI_LINEAR = 0
PHI_MEAN = 1
SCORE_CMP_OVERLAP = 0
SCORE_MEAN_DOT = 1
BR_CMP = 1
BR_SLC = 2
BR_WIN = 4
BR_ALL = BR_CMP | BR_SLC | BR_WIN


@dataclasses.dataclass(frozen=True)
class NSAConfig:
    name: str
    batch: int
    seq_len: int
    num_kv_heads: int
    heads_per_group: int
    d_k: int
    d_v: int
    cmp_block: int
    cmp_stride: int
    slc_block: int
    top_n: int
    n_init: int
    n_local: int
    window: int
    phi: int = PHI_LINEAR
    score_mode: int = SCORE_CMP_OVERLAP
    branches: int = BR_ALL
    softmax_scale: float = 0.0  # 0 -> 1/sqrt(d_k)
    decode: bool = False        # one query per sequence at t = seq_len - 1
    fp32_inputs: bool = False   # the tiny case draws fp32 data (rounded to bf16 for the GPU)
    seed: int = 0

    # ---- derived sizes ----
    @property
    def num_heads(self) -> int:
        return self.num_kv_heads * self.heads_per_group

    @property
    def n_cmp(self) -> int:
        """Number of compressed blocks: floor((T - l) / s) + 1 (0 if T < l)."""
        if self.seq_len < self.cmp_block:
            return 0
        return (self.seq_len - self.cmp_block) // self.cmp_stride + 1

    @property
    def n_slc(self) -> int:
        """Number of selection blocks: ceil(T / l')."""
        return -(-self.seq_len // self.slc_block)

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.d_k)

    def replace(self, **kw) -> "NSAConfig":
        return dataclasses.replace(self, **kw)


TINY = NSAConfig("tiny", 1, 1024, 1, 4, 64, 64, 32, 16, 64, 4, 1, 2, 128,
                 fp32_inputs=True, seed=0)
P8K = NSAConfig("8k", 1, 8192, 4, 16, 192, 128, 32, 16, 64, 16, 1, 2, 512, seed=1)
P64K = NSAConfig("64k", 1, 65536, 4, 16, 192, 128, 32, 16, 64, 16, 1, 2, 512, seed=2)
DECODE = NSAConfig("decode", 32, 65536, 4, 16, 192, 128, 32, 16, 64, 16, 1, 2, 512,
                   decode=True, seed=3)
MOBA = NSAConfig("moba", 1, 131072, 8, 1, 128, 128, 512, 512, 512, 3, 0, 1, 0,
                 phi=PHI_MEAN, score_mode=SCORE_MEAN_DOT, branches=BR_SLC, seed=4)

CONFIGS = {c.name: c for c in (TINY, P8K, P64K, DECODE, MOBA)}
