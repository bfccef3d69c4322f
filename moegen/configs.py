"""Shapes and input recipes of the synthetic MoE layers.

This module holds data only (sizes, distributions, routing variants); it holds
none of the layer's arithmetic.  Both the GPU path and the CPU oracle read it.

The shapes follow the model families the pages name as served (Flyweight 0.2.0
wheel METADATA, the served-families table: Qwen 3 MoE, and "DeepSeek-shaped MoE"
for K2-Horizon); the expert formats Q8_0 and Q4_0 are the GGUF formats the
pages list among grouped routed-expert kernels (Flyweight 0.5.1, "Models and
formats").  Everything else (sizes, distributions, bias) is the workload recipe
recorded in the design notes.
"""

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

Q8_0 = "q8_0"
Q4_0 = "q4_0"
Q4_K = "q4_k"
Q6_K = "q6_k"
MXFP4 = "mxfp4"
F32 = "f32"
BF16 = "bf16"
SOFTMAX = "softmax"
SIGMOID = "sigmoid"

# bytes per 32-element block (Q4_K: 144 per 256-element super-block)
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_K: 18}
# bytes per 256-element super-block of the K-quants
SUPER_BYTES = {Q4_K: 144, Q6_K: 210}


def row_bytes(qtype: str, n: int) -> int:
    """Bytes a row of n elements takes (MXFP4: its codes and its share of the
    scales, which sit after the whole matrix's codes)."""
    if qtype == MXFP4:
        return n // 2 + n // 32
    if qtype in SUPER_BYTES:
        return n // 256 * SUPER_BYTES[qtype]
    return n // 32 * BLOCK_BYTES[qtype]


@dataclass(frozen=True)
class LayerConfig:
    cid: int                     # workload id; also part of every seed
    name: str
    hidden: int                  # H
    n_experts: int               # E
    top_k: int                   # k
    ffn: int                     # F (routed expert inner size)
    expert_q: str                # Q8_0 | Q4_0
    act_dtype: str               # F32 | BF16
    router_dtype: str            # F32 | BF16
    score: str                   # SOFTMAX | SIGMOID
    w_std: float                 # std of the fp32 weights before quantization
    router_std: float = 0.05
    shared_ffn: int = 0          # 0: no shared expert
    shared_q: str = Q8_0
    zipf: Optional[float] = None # per-expert logit bias b_e = -s*ln(e+1)
    tokens: Tuple[int, ...] = field(default=(1,))
    act_quant: str = "none"      # "mxfp8": MXFP8 expert activations (MXFP4 experts);
                                 # "int8": int8 expert activations (Q8_0 / Q4_0 experts)

    def with_(self, **kw):
        return replace(self, **kw)

    @property
    def expert_bytes(self):
        """Bytes of one routed expert (gate + up + down)."""
        return 3 * self.ffn * row_bytes(self.expert_q, self.hidden)

    @property
    def shared_bytes(self):
        if not self.shared_ffn:
            return 0
        return 3 * self.shared_ffn * row_bytes(self.shared_q, self.hidden)

    @property
    def router_bytes(self):
        return self.n_experts * self.hidden * (4 if self.router_dtype == F32 else 2)

    def act_bytes(self, T):
        return T * self.hidden * (4 if self.act_dtype == F32 else 2)


TINY = LayerConfig(0, "tiny", 256, 8, 2, 512, Q8_0, F32, F32, SOFTMAX, 0.02,
                   tokens=(4,))
QWEN3_DECODE = LayerConfig(1, "qwen3-moe-30b-a3b-shaped decode", 2048, 128, 8, 768,
                           Q4_0, BF16, BF16, SOFTMAX, 0.02, tokens=(1, 4, 16))
QWEN3_PREFILL = LayerConfig(2, "qwen3-moe-30b-a3b-shaped prefill zipf1.1", 2048, 128,
                            8, 768, Q4_0, BF16, BF16, SOFTMAX, 0.02, zipf=1.1,
                            tokens=(2048,))
DEEPSEEK = LayerConfig(3, "deepseek-shaped", 7168, 256, 8, 2048, Q4_0, BF16, BF16,
                       SIGMOID, 0.015, shared_ffn=2048, shared_q=Q8_0,
                       tokens=(1, 32, 4096))
SWEEP_Q8 = LayerConfig(4, "sweep q8_0", 4096, 64, 4, 1536, Q8_0, BF16, BF16, SOFTMAX,
                       0.02, tokens=tuple(2 ** i for i in range(14)))
SWEEP_Q4 = SWEEP_Q8.with_(name="sweep q4_0", expert_q=Q4_0)

CONFIGS = {0: TINY, 1: QWEN3_DECODE, 2: QWEN3_PREFILL, 3: DEEPSEEK, 4: SWEEP_Q8}
