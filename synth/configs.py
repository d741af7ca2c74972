"""Synthetic workloads: parameter-tensor lists and gradient recipes.

Each workload is a list of parameter tensors in the fused layout (qkv fused,
gate and up projections fused), the number of simulated workers W, the kept
fraction (1 - sparsity) as an exact rational, and the gradient distribution.
The evaluated sparsities, 90% and 99%, come from the abstract of "SCAPE:
Accurate and Efficient LLM Training with Extreme Sparse Communication"
(shd-paper.top page) and the Results section of the gist.science Technical
Summary; the model shapes stand in for GPT-345M and the Llama models the pages
train, with synthetic values (no dataset, no trained weights).

This module describes shapes and distributions only; it holds none of the
optimizer's arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class Tensor:
    name: str
    shape: Tuple[int, ...]

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


@dataclass(frozen=True)
class Workload:
    name: str
    tensors: Tuple[Tensor, ...]
    W: int
    keep_num: int
    keep_den: int
    steps: int
    seed: int
    # gradient recipe: "iid" (one sigma), "loguniform" (sigma per tensor in
    # [1e-5, 1e-2]) or "student2" (Student-t, 2 d.o.f., times t_scale)
    grad_kind: str
    sigma: float = 1e-3
    t_scale: float = 1e-3
    quantise_every: int = 0  # tensors with index % quantise_every == 0 are quantised
    param_sigma: float = 0.02
    P: int = 0  # ownership shards for the step's mask statistic (0 -> W)
    shard_P: int = 32  # partition used for the timed per-worker mask build
    beta1: float = 0.9
    beta2: float = 0.95
    lr: float = 1e-3
    eps: float = 1e-8
    weight_decay: float = 0.0

    @property
    def numel(self) -> int:
        return sum(t.numel for t in self.tensors)

    @property
    def layer_sizes(self) -> List[int]:
        return [t.numel for t in self.tensors]

    def quantised(self, tensor_index: int) -> bool:
        return self.quantise_every > 0 and tensor_index % self.quantise_every == 0

    def with_tensors(self, tensors, name: Optional[str] = None) -> "Workload":
        return replace(self, tensors=tuple(tensors), name=name or self.name)


def _gpt345m_tensors(n_layers: int = 24, h: int = 1024, f: int = 4096, v: int = 50304,
                     pos: int = 1024) -> List[Tensor]:
    ts = [Tensor("word_emb", (v, h)), Tensor("pos_emb", (pos, h))]
    for i in range(n_layers):
        p = f"l{i}."
        ts += [
            Tensor(p + "ln1.w", (h,)), Tensor(p + "ln1.b", (h,)),
            Tensor(p + "qkv.w", (3 * h, h)), Tensor(p + "qkv.b", (3 * h,)),
            Tensor(p + "proj.w", (h, h)), Tensor(p + "proj.b", (h,)),
            Tensor(p + "ln2.w", (h,)), Tensor(p + "ln2.b", (h,)),
            Tensor(p + "fc1.w", (f, h)), Tensor(p + "fc1.b", (f,)),
            Tensor(p + "fc2.w", (h, f)), Tensor(p + "fc2.b", (h,)),
        ]
    ts += [Tensor("final_ln.w", (h,)), Tensor("final_ln.b", (h,))]
    return ts


def _llama_tensors(n_layers: int, h: int, ffn: int, vocab: int = 32000) -> List[Tensor]:
    ts = [Tensor("emb", (vocab, h))]
    for i in range(n_layers):
        p = f"l{i}."
        ts += [
            Tensor(p + "attn_norm", (h,)), Tensor(p + "qkv", (3 * h, h)), Tensor(p + "o", (h, h)),
            Tensor(p + "mlp_norm", (h,)), Tensor(p + "gate_up", (2 * ffn, h)),
            Tensor(p + "down", (h, ffn)),
        ]
    ts += [Tensor("final_norm", (h,)), Tensor("lm_head", (vocab, h))]
    return ts


def _adversarial_tensors(n_blocks: int = 64, n_norms: int = 16, emb=(32000, 4096), mat: int = 2048,
                         norm: int = 1024) -> List[Tensor]:
    ts = [Tensor("emb", emb)]
    for i in range(n_blocks):
        ts.append(Tensor(f"b{i}.mat", (mat, mat)))
        ts += [Tensor(f"b{i}.norm{j}", (norm,)) for j in range(n_norms)]
    return ts


SINGLE = Workload(
    name="single-1024x1024", tensors=(Tensor("w", (1024, 1024)),), W=4, keep_num=1, keep_den=10,
    steps=5, seed=1001, grad_kind="iid", sigma=1e-3)

GPT345M = Workload(
    name="gpt-345m", tensors=tuple(_gpt345m_tensors()), W=8, keep_num=1, keep_den=10, steps=5,
    seed=1002, grad_kind="loguniform")

LLAMA055 = Workload(
    name="llama-0.55b", tensors=tuple(_llama_tensors(16, 1536, 4096)), W=8, keep_num=1,
    keep_den=100, steps=5, seed=1003, grad_kind="loguniform")

LLAMA175 = Workload(
    name="llama-1.75b", tensors=tuple(_llama_tensors(32, 2048, 5504)), W=4, keep_num=1,
    keep_den=100, steps=10, seed=1004, grad_kind="loguniform")

ADVERSARIAL = Workload(
    name="adversarial-ties", tensors=tuple(_adversarial_tensors()), W=32, keep_num=1,
    keep_den=1000, steps=5, seed=1005, grad_kind="student2", t_scale=1e-3, quantise_every=10)

WORKLOADS = {w.name: w for w in (SINGLE, GPT345M, LLAMA055, LLAMA175, ADVERSARIAL)}


def reduced(wl: Workload) -> Workload:
    """Same tensor kinds, ordering and gradient recipe at oracle-friendly sizes.

    Matrices shrink so that a full multi-step oracle run takes seconds, while
    every layer still spans several GPU tiles or ends in a ragged tile.
    """
    if wl.name == "gpt-345m":
        ts = _gpt345m_tensors(2, h=256, f=1024, v=2000, pos=256)
    elif wl.name == "llama-0.55b":
        ts = _llama_tensors(2, 384, 1024, vocab=1000)
    elif wl.name == "llama-1.75b":
        ts = _llama_tensors(2, 512, 1376, vocab=1000)
    elif wl.name == "adversarial-ties":
        ts = _adversarial_tensors(4, 16, emb=(1000, 1024), mat=512, norm=1024)
    else:
        ts = list(wl.tensors)
    return wl.with_tensors(ts, name=wl.name + "-small")


def ragged() -> Workload:
    """Edge-case layout: sizes that are not multiples of 64, a one-element layer,
    and a layer whose kept count rounds up from a fraction."""
    ts = [Tensor("a", (1000,)), Tensor("b", (37,)), Tensor("c", (1,)), Tensor("d", (64,)),
          Tensor("e", (4097,)), Tensor("f", (33, 65)), Tensor("g", (70000,))]
    return Workload(name="ragged", tensors=tuple(ts), W=3, keep_num=3, keep_den=100, steps=5,
                    seed=1099, grad_kind="loguniform")
