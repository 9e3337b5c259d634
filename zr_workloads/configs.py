"""The five synthetic workloads: tensor lists, rank, contribution counts,
value distributions and AdamW hyper-parameters.

Workload data only; no partitioning or update arithmetic lives here.  The
tensor lists stand in for the pages' example models:

* the 7B model on 4 GPUs of the ddp-to-zero blog (111qqz.com), ledger section;
* the 7.5B model on 64 GPUs of the Zero-3 parameter-partitioning article
  (hotelren.com), section on ZeRO stage 1/2/3 memory savings;
* the 1T-parameter model on 512 V100s of the DeepSpeed ZeRO-3 encyclopedia
  entry (baike.kuaisou.com), applications section.

Shapes of the Llama-style and GPT-style lists are a reading of the
stated dimensions (the pages list no tensors).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

# AdamW hyper-parameters of the ZeRO tutorial (cnhsyj.com), section 3.1.
ADAMW_DEFAULT = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@dataclass(frozen=True)
class Workload:
    name: str
    tensors: Tuple[Tuple[str, Tuple[int, ...]], ...]   # (name, shape) in registration order
    n_d: int
    rank: int
    n_contrib: int                 # simulated per-rank gradient contributions
    steps: Tuple[int, ...]         # AdamW step counters t applied in order
    m_std: float                   # exp_avg ~ N(0, m_std) (0 -> zeros)
    v_high: float                  # exp_avg_sq ~ U[0, v_high) (0 -> zeros)
    grad_std: float = 1e-3         # each contribution ~ N(0, grad_std), rounded to bf16
    master_std: float = 0.02       # fp32 master ~ N(0, master_std)
    hparams: dict = field(default_factory=lambda: dict(ADAMW_DEFAULT))
    seed: int = 0
    threshold: int = 100_000

    @property
    def numels(self) -> List[int]:
        out = []
        for _, shape in self.tensors:
            n = 1
            for d in shape:
                n *= d
            out.append(n)
        return out


def _mlp_tiny():
    return (("fc1.weight", (1024, 512)), ("fc1.bias", (512,)),
            ("fc2.weight", (512, 1024)), ("fc2.bias", (1024,)))


def _llama_7b(layers=32, hidden=4096, ffn=11008, vocab=32000):
    t = [("embed_tokens.weight", (vocab, hidden))]
    for i in range(layers):
        p = f"layers.{i}."
        t += [(p + "self_attn.q_proj.weight", (hidden, hidden)),
              (p + "self_attn.k_proj.weight", (hidden, hidden)),
              (p + "self_attn.v_proj.weight", (hidden, hidden)),
              (p + "self_attn.o_proj.weight", (hidden, hidden)),
              (p + "mlp.gate_proj.weight", (ffn, hidden)),
              (p + "mlp.up_proj.weight", (ffn, hidden)),
              (p + "mlp.down_proj.weight", (hidden, ffn)),
              (p + "input_layernorm.weight", (hidden,)),
              (p + "post_attention_layernorm.weight", (hidden,))]
    t += [("norm.weight", (hidden,)), ("lm_head.weight", (vocab, hidden))]
    return tuple(t)


def _gpt_7p5b(layers=36, hidden=4096, vocab=50304):
    t = [("wte.weight", (vocab, hidden))]
    for i in range(layers):
        p = f"h.{i}."
        t += [(p + "ln_1.weight", (hidden,)), (p + "ln_1.bias", (hidden,)),
              (p + "attn.qkv.weight", (3 * hidden, hidden)), (p + "attn.qkv.bias", (3 * hidden,)),
              (p + "attn.proj.weight", (hidden, hidden)), (p + "attn.proj.bias", (hidden,)),
              (p + "ln_2.weight", (hidden,)), (p + "ln_2.bias", (hidden,)),
              (p + "mlp.fc1.weight", (4 * hidden, hidden)), (p + "mlp.fc1.bias", (4 * hidden,)),
              (p + "mlp.fc2.weight", (hidden, 4 * hidden)), (p + "mlp.fc2.bias", (hidden,))]
    t += [("ln_f.weight", (hidden,)), ("ln_f.bias", (hidden,))]
    return tuple(t)


TINY_MLP = Workload(
    name="tiny_mlp_nd4_r0", tensors=_mlp_tiny(), n_d=4, rank=0, n_contrib=4,
    steps=(1,), m_std=0.0, v_high=0.0, seed=1)

FLAT_7B = Workload(
    name="flat_7e9_nd4_r0", tensors=(("flat", (7_000_000_000,)),), n_d=4, rank=0, n_contrib=4,
    steps=(10,), m_std=1e-4, v_high=1e-6, seed=2)

LLAMA_7B = Workload(
    name="llama7b_nd64_r17", tensors=_llama_7b(), n_d=64, rank=17, n_contrib=64,
    steps=(1,), m_std=0.0, v_high=0.0, seed=3)

GPT_7P5B = Workload(
    name="gpt7p5b_nd64_r0_10steps", tensors=_gpt_7p5b(), n_d=64, rank=0, n_contrib=8,
    steps=tuple(range(1, 11)), m_std=0.0, v_high=0.0, seed=4)

FLAT_1T = Workload(
    name="flat_1e12_nd512_r0", tensors=(("flat", (1_000_000_000_000,)),), n_d=512, rank=0,
    n_contrib=8, steps=(1000,), m_std=1e-4, v_high=1e-6,
    hparams=dict(ADAMW_DEFAULT, lr=1e-4, weight_decay=0.1), seed=5)

ALL = (TINY_MLP, FLAT_7B, LLAMA_7B, GPT_7P5B, FLAT_1T)
BY_NAME = {w.name: w for w in ALL}
