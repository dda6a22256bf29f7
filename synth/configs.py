"""Workload shapes for the ResidualKV hot path.

Five workloads, each a synthetic prototype-mixture KV cache:

  tiny        1 layer x 1 KV head, seq 1024, fp32, s=16, k=4, int8/g32.
              Small enough for the oracle to run whole.
  llama3_8b_layer
              one Llama-3-8B-shaped layer: 8 KV heads, 32 query heads,
              seq 8192, bf16, s=32, k=8, int4/g32, decode batch 1.
  llama3_8b_32k
              long-context decode: 32 layers x 8 KV heads, context 32768,
              batch 8, bf16, s=64, k=8, int4/g32.  Decode is timed per layer.
  dynamic_131k
              one layer, 8 KV heads, seq 131072, bf16, dynamic stride
              (base 16, doubling past 4096), k=8, int4/g32, drifting
              prototypes.
  prefill_stress
              28 layers x 4 KV heads (28 query heads), batch 16 x seq 16384,
              bf16, 30 % heavy-tailed tokens, s=32, k=16, group 64, int4 and
              int2.

The numbers of prototypes and the noise scales follow the workload
descriptions; where a description leaves them open (dynamic_131k,
prefill_stress) the values of the neighbouring workload are reused.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    index: int                  # 0-based position in the workload list
    n_layers: int
    n_kv_heads: int
    n_q_heads: int
    seq_len: int
    batch: int
    head_dim: int
    dtype: str                  # "f32" or "bf16"
    n_protos: int
    sigma: float
    stride_base: int
    double_after: int           # 0 = fixed stride
    k: int
    bits: Tuple[int, ...]       # residual code widths exercised
    group: int
    drift: float = 0.0          # random-walk step per drift block (0 = none)
    drift_block: int = 1024
    heavy_frac: float = 0.0     # fraction of Student-t tokens
    heavy_nu: int = 3
    decode: bool = True

    @property
    def n_inst(self) -> int:
        """Independent sequences x layers; each instance has its own cache."""
        return self.n_layers * self.batch

    @property
    def head_tokens(self) -> int:
        return self.n_inst * self.n_kv_heads * self.seq_len


CONFIGS = (
    Config("tiny", 0, n_layers=1, n_kv_heads=1, n_q_heads=1, seq_len=1024,
           batch=1, head_dim=128, dtype="f32", n_protos=64, sigma=0.1,
           stride_base=16, double_after=0, k=4, bits=(8,), group=32),
    Config("llama3_8b_layer", 1, n_layers=1, n_kv_heads=8, n_q_heads=32,
           seq_len=8192, batch=1, head_dim=128, dtype="bf16", n_protos=512,
           sigma=0.2, stride_base=32, double_after=0, k=8, bits=(4,),
           group=32),
    Config("llama3_8b_32k", 2, n_layers=32, n_kv_heads=8, n_q_heads=32,
           seq_len=32768, batch=8, head_dim=128, dtype="bf16", n_protos=2048,
           sigma=0.15, stride_base=64, double_after=0, k=8, bits=(4,),
           group=32),
    Config("dynamic_131k", 3, n_layers=1, n_kv_heads=8, n_q_heads=32,
           seq_len=131072, batch=1, head_dim=128, dtype="bf16",
           n_protos=2048, sigma=0.15, stride_base=16, double_after=4096,
           k=8, bits=(4,), group=32, drift=0.01, drift_block=1024),
    Config("prefill_stress", 4, n_layers=28, n_kv_heads=4, n_q_heads=28,
           seq_len=16384, batch=16, head_dim=128, dtype="bf16", n_protos=512,
           sigma=0.2, stride_base=32, double_after=0, k=16, bits=(4, 2),
           group=64, heavy_frac=0.3, heavy_nu=3, decode=False),
)


def get_config(name_or_index) -> Config:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    for c in CONFIGS:
        if c.name == name_or_index:
            return c
    raise KeyError(name_or_index)
