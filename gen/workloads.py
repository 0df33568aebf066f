"""Named synthetic workloads: shapes, value laws and seeds.

Shapes follow the linear layers of Llama-2-7B and Llama-2-70B, the model
families the AWQ summary page (fdeinterviews.com, paragraph 4) reports on; the
weights are random, since no trained checkpoint is used.  A layer is (K, N):
K input channels (the contraction), N output channels; W is [N][K] like a
torch Linear weight.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple


def seed_for(workload_id: int, tensor_id: int) -> int:
    """Seed of one tensor: 1000 * workload id + tensor id."""
    return 1000 * int(workload_id) + int(tensor_id)


@dataclass(frozen=True)
class Layer:
    name: str
    K: int
    N: int
    sigma_w: float


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    layers: Tuple[Layer, ...]
    batch: Tuple[int, ...]
    group: int = 128
    n_alpha: int = 20
    calib_rows: int = 0
    lognormal: bool = False
    notes: str = ""
    extra: Dict[str, object] = field(default_factory=dict)


_L7 = (
    Layer("q_proj", 4096, 4096, 0.02),
    Layer("k_proj", 4096, 4096, 0.02),
    Layer("v_proj", 4096, 4096, 0.02),
    Layer("o_proj", 4096, 4096, 0.02),
    Layer("gate_proj", 4096, 11008, 0.02),
    Layer("up_proj", 4096, 11008, 0.02),
    Layer("down_proj", 11008, 4096, 0.02),
)

_L70 = (
    Layer("qkv_proj", 8192, 10240, 0.015),
    Layer("o_proj", 8192, 8192, 0.015),
    Layer("gate_proj", 8192, 28672, 0.015),
    Layer("up_proj", 8192, 28672, 0.015),
    Layer("down_proj", 28672, 8192, 0.015),
)

WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload(1, "single_layer_512", (Layer("linear", 512, 512, 0.02),), (1, 4),
                 calib_rows=64,
                 notes="W 512x512 N(0,0.02^2); X 64x512 N(0,1), 1% channels x20; 20 alphas; gemm at M=1,4"),
        Workload(2, "llama2_7b_decode_m1", _L7, (1,),
                 notes="7 decode GEMVs of one Llama-2-7B block at M=1"),
        Workload(3, "batch_sweep_4096x11008", (Layer("gate_proj", 4096, 11008, 0.02),),
                 (1, 2, 4, 8, 16, 64, 256, 1024),
                 notes="one K=4096, N=11008 layer over M in {1..1024}"),
        Workload(4, "llama2_70b_layers", _L70, (1, 8, 16),
                 notes="Llama-2-70B-shaped layers at M=1,8,16"),
        Workload(5, "llama2_7b_block_search", _L7, (),
                 calib_rows=65536, lognormal=True,
                 notes="awq_quantize over the 7 linears of a 7B block; 65,536 calibration rows "
                       "with a lognormal channel profile and 1% outliers x20"),
    )
}


def layer_inputs_7b_block() -> List[Tuple[str, str]]:
    """Which calibration input feeds each 7B linear (q/k/v share one input, gate/up another)."""
    return [("q_proj", "attn_in"), ("k_proj", "attn_in"), ("v_proj", "attn_in"),
            ("o_proj", "o_in"), ("gate_proj", "mlp_in"), ("up_proj", "mlp_in"),
            ("down_proj", "down_in")]
