"""The five synthetic workloads the library is tested and measured on.

Shapes follow the workloads the pages name (GPT-2 at sequence length 1K, BERT-large,
16K-long sequences; reading card section 4, results table) plus a one-head fp32 case and a
decode step (the dataflow essay's evaluation checklist asks for prefill and decode to be
measured apart). No dataset is read: every tensor is drawn from a seeded generator.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "bf16" or "fp32": the element type of Q, K, V and O
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    input_std: float      # Q/K/V are input_std * N(0, 1) before rounding to dtype
    lengths: Optional[Tuple[int, int]]  # inclusive range of per-sequence valid key counts
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def counted_flops(self) -> int:
        """4*B*H*Nq*Nk*d, halved for causal masking (the counting convention of the target)."""
        f = 4 * self.B * self.H * self.Nq * self.Nk * self.d
        return f // 2 if self.causal else f


SINGLE_HEAD_FP32 = Workload("single_head_fp32_n128_d64", "fp32", 1, 1, 128, 128, 64,
                            False, 1.0, None, 1001)
GPT2_SMALL_CAUSAL = Workload("gpt2s_causal_b8_h12_n1024_d64", "bf16", 8, 12, 1024, 1024, 64,
                             True, 1.0, None, 1002)
BERT_LARGE_PADDED = Workload("bertl_padded_b16_h16_n512_d64", "bf16", 16, 16, 512, 512, 64,
                             False, 1.0, (128, 512), 1003)
LONG_CAUSAL_16K = Workload("long_causal_b2_h16_n16384_d128", "bf16", 2, 16, 16384, 16384, 128,
                           True, 0.5, None, 1004)
DECODE_SPLIT_KV = Workload("decode_b64_h32_nk8192_d128", "bf16", 64, 32, 1, 8192, 128,
                           False, 1.0, (1024, 8192), 1005)

ALL = (SINGLE_HEAD_FP32, GPT2_SMALL_CAUSAL, BERT_LARGE_PADDED, LONG_CAUSAL_16K, DECODE_SPLIT_KV)
BY_NAME = {w.name: w for w in ALL}
