"""Seeded synthetic inputs for the sparse-MoE decode layer.

This module is shared by the CPU oracle, the tests and the benchmark.  It
holds NO arithmetic of the method (no routing, no activation, no masking, no
projection): it only draws random tensors of the workloads' shapes and value
distributions and, for bf16 layers, rounds them once to bf16 bit patterns.

Workloads (layer shapes) are the MoE families the intra-expert-sparsity page
analyses in its technical summary (Methodology, empirical analysis: Granite,
OLMoE, DeepSeek-V2, GPT-OSS, Qwen, Llama-4).  Their real weights are not
available, so each layer is a random-init layer of that shape:

* expert weights ~ N(0, 1/fan_in): fan_in = hidden for gate/up, d_ff for down;
* router weights ~ N(0, 1/hidden);
* tokens x ~ N(0, 1);
* an optional per-expert router bias b[e] = -a*ln(e+1) (Zipf(a) load skew).

Weight layout (the library's ABI): gate, up and down are all [E, d_ff, H]
row-major, i.e. neuron-major.  Row j of the down matrix is neuron j's
H-vector contribution to the output (a torch ``down_proj.weight`` [H, d_ff]
is its transpose).  The router matrix is [E, H].

Every tensor is drawn from its own numpy ``SeedSequence([seed, matrix_id,
expert, group])`` stream, so one expert can be generated alone, in any
order, on any thread, with identical bits.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

# matrix ids of the SeedSequence keys
_GATE, _UP, _DOWN, _ROUTER, _TOKENS = 1, 2, 3, 4, 5
# expert groups of the SeedSequence keys
ROUTED, SHARED = 0, 1


@dataclass(frozen=True)
class LayerShape:
    """Geometry and input recipe of one synthetic MoE layer."""

    name: str
    hidden: int
    n_experts: int
    d_ff: int
    top_k: int
    norm_topk: bool
    dtype: str                       # "f32" or "bf16": x, router and expert weights
    n_shared: int = 0                # always-on shared experts
    d_ff_shared: int = 0
    zipf_bias: Optional[float] = None  # a of b[e] = -a*ln(e+1), or None
    batches: tuple = ()              # token counts the workload is run at
    sparsities: tuple = (0.9,)       # routed-expert sparsities it is run at
    shared_sparsities: tuple = ()    # shared-expert sparsities it is run at
    note: str = field(default="", compare=False)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)


# The five layer workloads.  Names say what each layer is; sizes are the
# families' published layer shapes.
LAYERS = {
    "tiny-f32": LayerShape(
        name="tiny-f32", hidden=256, n_experts=8, d_ff=512, top_k=2,
        norm_topk=False, dtype="f32", batches=(4,), sparsities=(0.9,),
        note="single fp32 layer, top-2 softmax routing, parity only"),
    "olmoe-like": LayerShape(
        name="olmoe-like", hidden=2048, n_experts=64, d_ff=1024, top_k=8,
        norm_topk=False, dtype="bf16", batches=(1, 4, 16),
        sparsities=(0.0, 0.5, 0.75, 0.9),
        note="OLMoE-like layer, no shared expert"),
    "qwen3-moe-like": LayerShape(
        name="qwen3-moe-like", hidden=2048, n_experts=128, d_ff=768, top_k=8,
        norm_topk=True, dtype="bf16", zipf_bias=1.1,
        batches=(1, 2, 4, 8, 16, 32, 64), sparsities=(0.9,),
        note="Qwen3-MoE-like layer, normalised top-k weights, Zipf(1.1) router bias"),
    "deepseek-v2-like": LayerShape(
        name="deepseek-v2-like", hidden=5120, n_experts=160, d_ff=1536, top_k=6,
        norm_topk=False, dtype="bf16", n_shared=2, d_ff_shared=1536,
        batches=(1, 2, 4, 8, 16, 32), sparsities=(0.9,), shared_sparsities=(0.0, 0.5),
        note="DeepSeek-V2-like layer, 2 always-on shared experts"),
    "llama4-like": LayerShape(
        name="llama4-like", hidden=5120, n_experts=16, d_ff=8192, top_k=1,
        norm_topk=False, dtype="bf16", n_shared=1, d_ff_shared=8192,
        batches=(1, 8, 64, 256, 1024), sparsities=(0.9,), shared_sparsities=(0.9,),
        note="Llama-4-like large-expert layer, 1 shared expert"),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, matrix: int, expert: int = 0, group: int = ROUTED):
    return np.random.default_rng(np.random.SeedSequence([seed, matrix, expert, group]))


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite by construction (normal draws)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _draw(rng, shape, std: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a if dtype == "f32" else round_to_bf16_bits(a)


def expert_matrix(shape: LayerShape, seed: int, which: str, e: int,
                  group: int = ROUTED) -> np.ndarray:
    """One expert's gate/up/down matrix, [d_ff, H] neuron-major.

    Returns float32 for an f32 layer, uint16 bf16 bits for a bf16 layer."""
    d_ff = shape.d_ff if group == ROUTED else shape.d_ff_shared
    mid = {"gate": _GATE, "up": _UP, "down": _DOWN}[which]
    fan_in = shape.hidden if which in ("gate", "up") else d_ff
    return _draw(_rng(seed, mid, e, group), (d_ff, shape.hidden),
                 1.0 / np.sqrt(fan_in), shape.dtype)


def expert_weights(shape: LayerShape, seed: int = 0, group: int = ROUTED,
                   experts=None, threads: Optional[int] = None):
    """Stacked (gate, up, down), each [n, d_ff, H], for the listed experts
    (default: all experts of the group)."""
    n_all = shape.n_experts if group == ROUTED else shape.n_shared
    d_ff = shape.d_ff if group == ROUTED else shape.d_ff_shared
    experts = list(range(n_all)) if experts is None else list(experts)
    np_dtype = np.float32 if shape.dtype == "f32" else np.uint16
    out = [np.empty((len(experts), d_ff, shape.hidden), dtype=np_dtype) for _ in range(3)]

    def job(arg):
        i, e = arg
        for m, which in enumerate(("gate", "up", "down")):
            out[m][i] = expert_matrix(shape, seed, which, e, group)

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(job, enumerate(experts)))
    return tuple(out)


class LazyExperts:
    """Indexable view ``w[e]`` of one matrix kind that draws expert e on use.

    Lets a CPU consumer touch only the experts it needs on layers whose
    full weights would not fit host memory comfortably."""

    def __init__(self, shape: LayerShape, seed: int, which: str, group: int = ROUTED):
        self.shape, self.seed, self.which, self.group = shape, seed, which, group
        n = shape.n_experts if group == ROUTED else shape.n_shared
        d = shape.d_ff if group == ROUTED else shape.d_ff_shared
        self.n = n
        self.item_shape = (d, shape.hidden)
        self.dtype = np.float32 if shape.dtype == "f32" else np.uint16

    def __len__(self):
        return self.n

    def __getitem__(self, e):
        if not 0 <= e < self.n:
            raise IndexError(e)
        return expert_matrix(self.shape, self.seed, self.which, e, self.group)


def router_matrix(shape: LayerShape, seed: int = 0) -> np.ndarray:
    """Router weights [E, H] ~ N(0, 1/H)."""
    return _draw(_rng(seed, _ROUTER), (shape.n_experts, shape.hidden),
                 1.0 / np.sqrt(shape.hidden), shape.dtype)


def router_bias(shape: LayerShape) -> Optional[np.ndarray]:
    """Per-expert router-logit bias [E] fp32 giving Zipf(a) skew, or None.

    b[e] = -a*ln(e+1): exp(b) is proportional to the Zipf(a) mass of rank
    e+1, so expert 0 is the hottest."""
    if shape.zipf_bias is None:
        return None
    e = np.arange(shape.n_experts, dtype=np.float64)
    return (-shape.zipf_bias * np.log1p(e)).astype(np.float32)


def tokens(shape: LayerShape, seed: int, T: int) -> np.ndarray:
    """Token batch [T, H] ~ N(0, 1) (f32, or bf16 bits)."""
    return _draw(_rng(seed, _TOKENS, T), (T, shape.hidden), 1.0, shape.dtype)
