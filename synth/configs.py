"""Workload registry: the five single-layer prefill shapes.

Shapes follow the Llama-3.1-8B (32 query heads, 8 KV heads, head_dim 128,
RoPE base 5e5) and Qwen2.5-7B (28/4/128, RoPE base 1e6) attention layers that
the ProxyAttn blog post (ir.hit.edu.cn, section 5 "实验结果") evaluates on; the
block size is the 128x128 tile of its section 2 ("为什么必须是 Block-wise").
Lengths span 2K (tiny oracle case) to 256K.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    num_heads: int          # H, query heads
    num_kv_heads: int       # Hkv
    head_dim: int           # d
    seq_len: int            # N
    num_proxies: int        # G
    gammas: Tuple[float, ...]
    seed: int
    rope_base: Optional[float]     # None: no rotary embedding
    beta_range: Tuple[float, float]  # per-head sharpness, log-uniform
    n_needles: int
    needle_query_frac: float
    group_latent_corr: Optional[float] = None  # per-KV-head latent, correlation between heads
    dtype: str = "bf16"     # storage type of the generated tensors
    block: int = 128
    description: str = ""

    @property
    def gamma(self) -> float:
        return self.gammas[-1]

    @property
    def nb(self) -> int:
        return -(-self.seq_len // self.block)     # the last block may be partial

    def with_(self, **kw) -> "WorkloadConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny_d64_2k": WorkloadConfig(
        name="tiny_d64_2k", num_heads=4, num_kv_heads=2, head_dim=64, seq_len=2048,
        num_proxies=2, gammas=(0.95,), seed=0, rope_base=None,
        beta_range=(0.5, 4.0), n_needles=8, needle_query_frac=0.10, dtype="fp32",
        description="tiny fp32, GQA 4/2, d=64, N=2048, G=2"),
    "llama8b_32k_g1": WorkloadConfig(
        name="llama8b_32k_g1", num_heads=32, num_kv_heads=8, head_dim=128, seq_len=32768,
        num_proxies=1, gammas=(0.95,), seed=1, rope_base=500000.0,
        beta_range=(0.5, 4.0), n_needles=64, needle_query_frac=0.10,
        description="Llama-3.1-8B layer, N=32K, G=1"),
    "llama8b_128k_g4": WorkloadConfig(
        name="llama8b_128k_g4", num_heads=32, num_kv_heads=8, head_dim=128, seq_len=131072,
        num_proxies=4, gammas=(0.95,), seed=2, rope_base=500000.0,
        beta_range=(0.5, 4.0), n_needles=256, needle_query_frac=0.05,
        description="Llama-3.1-8B layer, N=128K, G=4"),
    "qwen7b_64k_g4": WorkloadConfig(
        name="qwen7b_64k_g4", num_heads=28, num_kv_heads=4, head_dim=128, seq_len=65536,
        num_proxies=4, gammas=(0.9,), seed=3, rope_base=1000000.0,
        beta_range=(0.5, 6.0), n_needles=128, needle_query_frac=0.05,
        group_latent_corr=0.3,
        description="Qwen2.5-7B layer, N=64K, G=4 (one proxy per GQA group)"),
    "long_256k_g8": WorkloadConfig(
        name="long_256k_g8", num_heads=32, num_kv_heads=8, head_dim=128, seq_len=262144,
        num_proxies=8, gammas=(0.8, 0.9, 0.95), seed=4, rope_base=500000.0,
        beta_range=(1.0, 8.0), n_needles=512, needle_query_frac=0.02,
        description="long stress case, N=256K, G=8"),
}


def get_config(name: str) -> WorkloadConfig:
    return CONFIGS[name]
