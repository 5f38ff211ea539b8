"""Workload shapes for the ZeRO-1 step: tensor lists and the five configurations.

Model names are tensor SHAPES only (no weights, no data): GPT-2 small and
Llama-7B parameter lists in their usual module order, flattened in list order
into one vector that W data-parallel ranks cut into equal contiguous shards
(rank r owns flat elements [r*S, (r+1)*S), S = ceil(N/W)).
"""
from __future__ import annotations

from dataclasses import dataclass, field


def gpt2_small_tensors(n_layer=12, d=768, ffn=3072, vocab=50257, n_ctx=1024):
    """GPT-2 small parameter list (tied LM head): 148 tensors, 124,439,808 elements."""
    t = [("wte", vocab * d), ("wpe", n_ctx * d)]
    for i in range(n_layer):
        p = f"h.{i}."
        t += [(p + "ln_1.weight", d), (p + "ln_1.bias", d),
              (p + "attn.c_attn.weight", d * 3 * d), (p + "attn.c_attn.bias", 3 * d),
              (p + "attn.c_proj.weight", d * d), (p + "attn.c_proj.bias", d),
              (p + "ln_2.weight", d), (p + "ln_2.bias", d),
              (p + "mlp.c_fc.weight", d * ffn), (p + "mlp.c_fc.bias", ffn),
              (p + "mlp.c_proj.weight", ffn * d), (p + "mlp.c_proj.bias", d)]
    t += [("ln_f.weight", d), ("ln_f.bias", d)]
    return t


def llama_7b_tensors(n_layer=32, d=4096, ffn=11008, vocab=32000):
    """Llama-7B parameter list (untied LM head): 291 tensors, 6,738,415,616 elements."""
    t = [("embed_tokens", vocab * d)]
    for i in range(n_layer):
        p = f"layers.{i}."
        t += [(p + "self_attn.q_proj", d * d), (p + "self_attn.k_proj", d * d),
              (p + "self_attn.v_proj", d * d), (p + "self_attn.o_proj", d * d),
              (p + "mlp.gate_proj", d * ffn), (p + "mlp.up_proj", d * ffn),
              (p + "mlp.down_proj", ffn * d),
              (p + "input_layernorm", d), (p + "post_attention_layernorm", d)]
    t += [("norm", d), ("lm_head", vocab * d)]
    return t


def shard_range(n_total: int, W: int, rank: int):
    """[begin, end) of rank's contiguous shard; S = ceil(N/W), the last shard may be short."""
    S = -(-n_total // W)
    b = min(rank * S, n_total)
    e = min(b + S, n_total)
    return b, e


@dataclass
class Config:
    name: str
    workload: str
    W: int
    rank: int
    sigma: float
    outlier_pct: int
    steps: int
    tensors: list = field(default_factory=list)   # [(name, numel)]; one tensor for flat configs
    all_replicas_resident: bool = False          # True: every replica's full gradient is in HBM
    mv_bf16: bool = False
    seed: int = 0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    max_norm: float = 1.0
    master_sigma: float = 0.02
    parity_ranks: tuple = ()

    @property
    def n_total(self) -> int:
        return sum(n for _, n in self.tensors)

    @property
    def shard(self):
        return shard_range(self.n_total, self.W, self.rank)

    @property
    def S(self) -> int:
        b, e = self.shard
        return e - b

    def hparams(self, t: int) -> dict:
        return dict(lr=self.lr, beta1=self.beta1, beta2=self.beta2, eps=self.eps,
                    weight_decay=self.weight_decay, max_norm=self.max_norm, step=t)

    @property
    def bytes_per_param(self) -> int:
        """Algorithmic HBM bytes per shard element: W bf16 grad reads, master/m/v
        read+write (24 B, or 8+8 with bf16 moments) and the bf16 param write."""
        return 2 * self.W + (18 if self.mv_bf16 else 26)


def configs():
    c = {}
    c["C1"] = Config("C1", "flat 2^20 params, W=4, rank 0", W=4, rank=0, sigma=1e-3,
                     outlier_pct=0, steps=10, tensors=[("flat", 1 << 20)],
                     all_replicas_resident=True, seed=0x5EED0001, parity_ranks=(0, 1, 2, 3))
    c["C2"] = Config("C2", "GPT-2 small (124,439,808 params, 148 tensors), W=8, rank 4",
                     W=8, rank=4, sigma=1e-2, outlier_pct=1, steps=10,
                     tensors=gpt2_small_tensors(), all_replicas_resident=True,
                     seed=0x5EED0002, parity_ranks=tuple(range(8)))
    c["C3"] = Config("C3", "dense 7.5e9 params, W=64, rank 0", W=64, rank=0, sigma=1e-3,
                     outlier_pct=0, steps=10, tensors=[("flat", 7_500_000_000)],
                     seed=0x5EED0003, parity_ranks=(0,))
    c["C4"] = Config("C4", "Llama-7B (6,738,415,616 params, 291 tensors), W=8, rank 3",
                     W=8, rank=3, sigma=1e-3, outlier_pct=0, steps=5,
                     tensors=llama_7b_tensors(), seed=0x5EED0004, parity_ranks=(3, 0))
    c["C5a"] = Config("C5a", "dense 7e9 params, W=1 (full AdamW step), fp32 m,v", W=1, rank=0,
                      sigma=1e-3, outlier_pct=0, steps=3, tensors=[("flat", 7_000_000_000)],
                      seed=0x5EED0005, parity_ranks=(0,))
    c["C5b"] = Config("C5b", "dense 7e9 params, W=1 (full AdamW step), bf16 m,v", W=1, rank=0,
                      sigma=1e-3, outlier_pct=0, steps=3, tensors=[("flat", 7_000_000_000)],
                      mv_bf16=True, seed=0x5EED0005, parity_ranks=(0,))
    return c
