"""The five workloads of the CSA/HCA hot path, plus the 128K CSA prefill.

Constants come from the pages: block size m = 4 and m' = 128, top-k 512
(Flash) / 1024 (Pro), a 128-token sliding window (kenelite analysis, spec table
in section 2 and sections 5-7; llm-tech overview, CSA and HCA sections), FP8
KV with BF16 RoPE dims and an FP4 indexer (llm-tech overview, "other
architecture details").  Shapes the pages leave open (head counts, head dim,
indexer dims) are the stated workload recipe.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    kind: str            # "csa_prefill" | "hca_prefill" | "csa_decode" | "hybrid_decode"
    B: int               # batch
    T: int               # prefill: tokens; decode: cached context length
    H: int               # query heads
    D: int               # shared K/V head dim
    R: int               # trailing RoPE dims stored in BF16
    m: int               # CSA block size (or m' for HCA prefill)
    k: int               # top-k (0 for HCA)
    W: int               # sliding window
    H_I: int = 0         # indexer heads
    d_I: int = 0         # indexer head dim
    kv_fmt: str = "fp8"  # "f32" | "fp8" (bulk E4M3 + BF16 RoPE)
    idx_fmt: str = "fp8"  # "f32" | "fp8" | "mxfp4"
    act_fmt: str = "bf16"  # token / query activation dtype: "f32" | "bf16"
    m_hca: int = 128     # HCA block size for the hybrid decode layer
    rmsnorm: bool = True
    seed: int = 0

    @property
    def N(self) -> int:
        """Number of complete blocks (compressed entries) per sequence."""
        return self.T // self.m

    @property
    def N_hca(self) -> int:
        return self.T // self.m_hca

    def scaled(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # Tiny fp32 CSA: raw N(0,1) activations, weights N(0, 0.02^2).
    "tiny_csa_f32": Config("tiny_csa_f32", "csa_prefill", B=1, T=2048, H=4, D=64, R=16, m=4,
                           k=64, W=128, H_I=2, d_I=32, kv_fmt="f32", idx_fmt="f32",
                           act_fmt="f32", rmsnorm=False),
    # Flash-like CSA prefill, 32K tokens.
    "csa_prefill_32k": Config("csa_prefill_32k", "csa_prefill", B=1, T=32768, H=64, D=512,
                              R=64, m=4, k=512, W=128, H_I=8, d_I=64),
    # The same CSA layer at 128K tokens (the prefill length of the headline metric).
    "csa_prefill_128k": Config("csa_prefill_128k", "csa_prefill", B=1, T=131072, H=64, D=512,
                               R=64, m=4, k=512, W=128, H_I=8, d_I=64),
    # HCA dense prefill at 128K tokens: m' = 128 -> 1024 entries.
    "hca_prefill_128k": Config("hca_prefill_128k", "hca_prefill", B=1, T=131072, H=64, D=512,
                               R=64, m=128, k=0, W=128),
    # Pro-like CSA decode at 1M context (262,144 entries per sequence).
    "csa_decode_1m": Config("csa_decode_1m", "csa_decode", B=32, T=1 << 20, H=128, D=512,
                            R=64, m=4, k=1024, W=128, H_I=8, d_I=64),
    # Hybrid CSA (MXFP4 indexer) + HCA decode at 1M context.
    "hybrid_decode_1m": Config("hybrid_decode_1m", "hybrid_decode", B=16, T=1 << 20, H=128,
                               D=512, R=64, m=4, k=1024, W=128, H_I=8, d_I=64,
                               idx_fmt="mxfp4", m_hca=128),
}

WEIGHT_STD = 0.02  # compressor gate/bias and indexer head weights


def get_config(name: str) -> Config:
    return CONFIGS[name]
