"""The five synthetic matrix sets the batched Muon step is checked and timed on.

Shapes follow ``nn.Linear.weight`` convention, ``(out_features, in_features)``,
row-major.  Sources of each set:

* ``tinymlp_f32`` -- the TinyMLP model of the DMuon quickstart page (``model.py``:
  d=512, ff=2048, four layers of gate/up/down projections).
* ``spectrum`` -- singular-spectrum-controlled matrices for the Newton-Schulz
  step sweep {3, 5, 7, 10} of the DMuon blog post ("N-S 步数选择").
* ``square4096`` -- the 4096x4096 matrix size the blog post uses for its
  vanilla-Muon time breakdown ("分布式 Muon 的性能瓶颈").
* ``llama3_8b`` -- projections of a Llama-3-8B-shaped transformer (the training
  guide's "standard Transformer (Llama, Qwen, Mistral)" predicate pattern).
* ``hybrid`` -- a GateDelta / hybrid-attention shaped model whose tiny
  ``a_proj``/``b_proj`` fall under the training guide's ``numel() < 100_000``
  exclusion and so take the elementwise-only route.

Values are drawn per matrix from independent seeded streams (see ``gen.py``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

ROOT_SEED = 42  # the quickstart scripts seed with torch.manual_seed(42)


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    rows: int
    cols: int

    @property
    def numel(self) -> int:
        return self.rows * self.cols


@dataclass(frozen=True)
class SetConfig:
    key: str
    cfg_id: int            # enters the seed sequence
    matrices: Tuple[MatrixSpec, ...]
    dtype: str             # "f32" or "bf16": grads and params
    grad_dist: str         # "normal" | "student_t3" | "spectrum"
    grad_scale: float      # std (normal) or multiplier (student_t3)
    weight_scale: float    # weights ~ N(0, weight_scale^2)
    momentum: float = 0.95
    nesterov: bool = True
    ns_steps: Tuple[int, ...] = (5,)
    lr: float = 0.02
    ns_only: bool = False  # set uses ns_batched (no momentum / update)
    extra_dtypes: Tuple[str, ...] = field(default_factory=tuple)

    @property
    def count(self) -> int:
        return len(self.matrices)

    def total_numel(self) -> int:
        return sum(m.numel for m in self.matrices)


def _layers(n_layers: int, per_layer: List[Tuple[str, int, int]]) -> Tuple[MatrixSpec, ...]:
    out = []
    for layer in range(n_layers):
        for name, r, c in per_layer:
            out.append(MatrixSpec(f"layers.{layer}.{name}", r, c))
    return tuple(out)


TINYMLP = SetConfig(
    key="tinymlp_f32", cfg_id=1,
    matrices=_layers(4, [("gate_proj", 2048, 512), ("up_proj", 2048, 512), ("down_proj", 512, 2048)]),
    dtype="f32", grad_dist="normal", grad_scale=1.0, weight_scale=1.0,
    ns_steps=(5,),
)

SPECTRUM = SetConfig(
    key="spectrum", cfg_id=2,
    matrices=tuple([MatrixSpec(f"wide.{i}", 256, 1024) for i in range(16)]
                   + [MatrixSpec(f"tall.{i}", 1024, 256) for i in range(16)]),
    dtype="f32", grad_dist="spectrum", grad_scale=1.0, weight_scale=0.0,
    ns_steps=(3, 5, 7, 10), ns_only=True, extra_dtypes=("bf16",),
)

SQUARE4096 = SetConfig(
    key="square4096", cfg_id=3,
    matrices=tuple(MatrixSpec(f"square.{i}", 4096, 4096) for i in range(64)),
    dtype="bf16", grad_dist="normal", grad_scale=1e-3, weight_scale=1.0,
    ns_steps=(5, 10),
)

LLAMA3_8B = SetConfig(
    key="llama3_8b", cfg_id=4,
    matrices=_layers(32, [
        ("self_attn.q_proj", 4096, 4096),
        ("self_attn.k_proj", 1024, 4096),
        ("self_attn.v_proj", 1024, 4096),
        ("self_attn.o_proj", 4096, 4096),
        ("mlp.gate_proj", 14336, 4096),
        ("mlp.up_proj", 14336, 4096),
        ("mlp.down_proj", 4096, 14336),
    ]),
    dtype="bf16", grad_dist="normal", grad_scale=1e-3, weight_scale=1.0,
    ns_steps=(5,),
)

HYBRID = SetConfig(
    key="hybrid", cfg_id=5,
    matrices=_layers(48, [
        ("attn.q_proj", 2048, 2048),
        ("attn.k_proj", 2048, 2048),
        ("attn.v_proj", 2048, 2048),
        ("attn.o_proj", 2048, 2048),
        ("mlp.gate_proj", 5632, 2048),
        ("mlp.up_proj", 5632, 2048),
        ("mlp.down_proj", 2048, 5632),
        ("attn.a_proj", 2048, 32),
        ("attn.b_proj", 2048, 32),
    ]),
    dtype="bf16", grad_dist="student_t3", grad_scale=1e-3, weight_scale=1.0,
    ns_steps=(5,),
)

CONFIGS = {c.key: c for c in (TINYMLP, SPECTRUM, SQUARE4096, LLAMA3_8B, HYBRID)}


def get_config(key: str) -> SetConfig:
    return CONFIGS[key]
