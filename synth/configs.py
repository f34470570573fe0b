"""Workload table: the five QE linear-layer configurations.

Shapes are those of the decoder-layer linears of Qwen2VL-2B, InternVL2-8B and
Qwen2VL-72B (the model families the Quant Experts paper evaluates, Tables 1-3),
plus one tiny single linear.  Hyper-parameters default to the paper's: total
SVD rank 64 split evenly between the shared and the routed experts (32 + 32),
N_r = 8 routed experts and k = 32 important channels per token (MCISLAB
DeepRead summary, "Method", last paragraph).
"""

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple


@dataclass(frozen=True)
class LinearSpec:
    name: str
    d_in: int
    d_out: int
    stream: str  # which activation tensor feeds this linear


@dataclass(frozen=True)
class ActRecipe:
    """Outlier structure of one activation stream.

    modalities: list of (n_tokens, n_fixed, fixed_mult, pool, n_per_token, tok_mult).
      n_fixed channels are scaled by fixed_mult on every token of the modality;
      each token additionally scales n_per_token distinct channels, drawn from a
      modality pool of `pool` channels (pool=0: all channels outside the fixed
      set), by tok_mult.  The channel sets of different modalities are disjoint.
    """

    modalities: Tuple[Tuple[int, int, float, int, int, float], ...]
    fixed_channels: Optional[Tuple[int, ...]] = None  # explicit fixed set (single modality)
    dtype: str = "bf16"


@dataclass(frozen=True)
class QEConfig:
    name: str
    seed: int
    T: int
    w_bits: int
    a_bits: int
    r_shared: int
    n_routed: int
    r_routed: int
    k: int
    linears: Tuple[LinearSpec, ...]
    acts: Dict[str, ActRecipe] = field(default_factory=dict)
    run_topk: bool = False
    description: str = ""

    def stream_dim(self, stream: str) -> int:
        for lin in self.linears:
            if lin.stream == stream:
                return lin.d_in
        raise KeyError(stream)

    def streams(self) -> List[str]:
        out: List[str] = []
        for lin in self.linears:
            if lin.stream not in out:
                out.append(lin.stream)
        return out


def _layer(hidden: int, kv: int, inter: int) -> Tuple[LinearSpec, ...]:
    return (
        LinearSpec("q", hidden, hidden, "x_attn"),
        LinearSpec("k", hidden, kv, "x_attn"),
        LinearSpec("v", hidden, kv, "x_attn"),
        LinearSpec("o", hidden, hidden, "x_o"),
        LinearSpec("gate", hidden, inter, "x_mlp"),
        LinearSpec("up", hidden, inter, "x_mlp"),
        LinearSpec("down", inter, hidden, "x_down"),
    )


def _streams(recipe: ActRecipe, names=("x_attn", "x_o", "x_mlp", "x_down")) -> Dict[str, ActRecipe]:
    return {n: recipe for n in names}


_C1 = QEConfig(
    name="tiny",
    seed=0,
    T=64,
    w_bits=4,
    a_bits=8,
    r_shared=8,
    n_routed=4,
    r_routed=8,
    k=8,
    linears=(LinearSpec("lin", 256, 512, "x"),),
    acts={"x": ActRecipe(modalities=((64, 2, 20.0, 0, 2, 10.0),), fixed_channels=(3, 17), dtype="f32")},
    run_topk=True,
    description="single QE linear 256->512, T=64, W4A8, fp32 activations",
)

_C2 = QEConfig(
    name="qwen2vl_2b",
    seed=1,
    T=2048,
    w_bits=4,
    a_bits=6,
    r_shared=32,
    n_routed=8,
    r_routed=32,
    k=32,
    linears=_layer(1536, 256, 8960),
    acts=_streams(ActRecipe(modalities=((1600, 4, 20.0, 64, 2, 10.0), (448, 4, 20.0, 64, 2, 10.0)))),
    description="Qwen2VL-2B-shaped layer linears, W4A6, 1600 image + 448 text tokens",
)

_C3 = QEConfig(
    name="internvl2_8b",
    seed=2,
    T=4096,
    w_bits=4,
    a_bits=8,
    r_shared=32,
    n_routed=8,
    r_routed=32,
    k=32,
    linears=_layer(4096, 1024, 14336),
    acts=_streams(ActRecipe(modalities=((4096, 8, 30.0, 0, 4, 15.0),))),
    run_topk=True,
    description="InternVL2-8B-shaped layer linears, W4A8, plus the channel top-k histogram",
)

_C4 = QEConfig(
    name="qwen2vl_72b",
    seed=3,
    T=4096,
    w_bits=4,
    a_bits=6,
    r_shared=32,
    n_routed=8,
    r_routed=32,
    k=32,
    linears=_layer(8192, 1024, 29568),
    acts=_streams(ActRecipe(modalities=((3200, 8, 30.0, 256, 4, 15.0), (896, 8, 30.0, 256, 4, 15.0)))),
    description="Qwen2VL-72B-shaped layer linears, W4A6 prefill, 3200 image + 896 text tokens",
)

_C5 = QEConfig(
    name="qwen2vl_72b_decode",
    seed=4,
    T=8,
    w_bits=3,
    a_bits=16,
    r_shared=32,
    n_routed=8,
    r_routed=32,
    k=32,
    linears=(LinearSpec("up", 8192, 29568, "x_mlp"), LinearSpec("down", 29568, 8192, "x_down")),
    # decode tokens follow the text-token pattern of the 72B prefill workload
    acts=_streams(ActRecipe(modalities=((8, 8, 30.0, 256, 4, 15.0),)), names=("x_mlp", "x_down")),
    description="Qwen2VL-72B-shaped MLP up/down in decode, T=8, W3A16 weight-only",
)

# The linear shapes of the listing's Table 8 (NPU speedups of QE over fp16 for Qwen2VL-7B
# linears in prefill at sequence length 128): IC x OC = 3584 x 3584, 3584 x 18944 and
# 18944 x 3584; the table covers W4A6, W4A8 and W3A16 (this default is W4A6).
_C6 = QEConfig(
    name="qwen2vl_7b_s128",
    seed=5,
    T=128,
    w_bits=4,
    a_bits=6,
    r_shared=32,
    n_routed=8,
    r_routed=32,
    k=32,
    linears=(LinearSpec("q", 3584, 3584, "x_attn"), LinearSpec("up", 3584, 18944, "x_mlp"),
             LinearSpec("down", 18944, 3584, "x_down")),
    acts=_streams(ActRecipe(modalities=((96, 4, 20.0, 64, 2, 10.0), (32, 4, 20.0, 64, 2, 10.0))),
                  names=("x_attn", "x_mlp", "x_down")),
    description="Qwen2VL-7B linear shapes of Table 8, prefill s=128 (96 image-like + 32 text-like tokens)",
)

CONFIGS: Dict[str, QEConfig] = {c.name: c for c in (_C1, _C2, _C3, _C4, _C5, _C6)}


def get_config(name: str) -> QEConfig:
    return CONFIGS[name]
