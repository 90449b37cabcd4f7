"""Seeded synthetic inputs for the quantized MoE expert layer.

This module is shared by the oracle-side tests and the GPU path.  It only draws
random numbers and lays them out; it holds none of the layer's arithmetic (no
routing, no quantization, no packing, no GEMM).  Everything it returns is an
*input*: activations, router logits (and an optional per-expert router bias),
full-precision expert weights and bf16 shared-expert weights.

Shapes follow the Inkling-Small model card ("wstewart3/Inkling-Small-W4A8-G128",
§1 "What is being created", settings table: hidden 4096, expert width 2048,
256 routed and 2 shared experts per sparse layer) and the row-FP8 Inkling-2-Small
card ("Inkling 2 Small FP8 for AMD MI300X", "Precision and files": scale tensors
of shape [384, output_channels], i.e. 384 routed experts).

Weight layout: w13 is [E, 2I, H] with the gate rows first and the up rows second
(the fused gate|up "w13" of "Inkling-512k-NVFP4-AQLM-hybrid", "On-disk tensor
format"); w2 is [E, H, I]; both in (out, in) orientation.

Every tensor comes from its own seeded torch generator, keyed by (seed, tensor id,
expert), so any single expert can be regenerated on its own.  The values depend
on the device the generator runs on: a test that compares the GPU path with the
oracle generates once and hands the *same* tensor to both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Iterator, Optional, Tuple

import numpy as np
import torch

__all__ = [
    "LayerConfig", "CONFIGS", "get_config", "tensor_seed", "make_activations",
    "router_weights", "make_router", "expert_weight", "hybrid_partition", "make_nvfp4_slabs",
    "make_aqlm_slabs", "iter_expert_weights", "make_shared_weights",
    "make_layer_inputs",
]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One synthetic MoE-layer workload."""
    name: str
    T: int                 # tokens
    H: int                 # hidden size
    I: int                 # expert width (intermediate)
    E: int                 # routed experts
    k: int                 # experts per token
    x_dtype: str           # "f32" or "bf16": dtype of the layer input x
    weight_format: str     # "w4a8" (INT4 g128), "w4a8_bf16s" (bf16 group scales) or "fp8row"
    router: str            # "matmul": logits = x @ Wr^T ; "gaussian": logits ~ N(0,1);
                           # "gumbel_zipf": logits = Gumbel(0,1), bias = -s*ln(rank)
    router_scale: float    # std of the router weights (matmul) -- unused otherwise
    zipf_s: float = 0.0    # Zipf exponent for "gumbel_zipf"
    n_shared: int = 0      # shared experts (bf16), each of width I
    x_scale: float = 1.0   # std of x
    w_std: float = 0.02    # std of expert weights
    seed: int = 17

    @property
    def R(self) -> int:
        return self.T * self.k


# The five workloads.  "tiny" is small enough for the oracle in seconds;
# "decode" and "prefill" are single Inkling-Small sparse layers; "skewed" adds
# Zipf-skewed routing and two bf16 shared experts; "fp8row" is the row-scaled
# FP8 expert variant with 384 experts.
CONFIGS = {
    "tiny": LayerConfig("tiny", T=16, H=256, I=128, E=8, k=2, x_dtype="f32",
                        weight_format="w4a8", router="matmul",
                        router_scale=1.0 / 16.0, x_scale=1.0 / 16.0),
    "decode": LayerConfig("decode", T=4, H=4096, I=2048, E=256, k=6, x_dtype="bf16",
                          weight_format="w4a8", router="gaussian", router_scale=0.0),
    "prefill": LayerConfig("prefill", T=2048, H=4096, I=2048, E=256, k=6, x_dtype="bf16",
                           weight_format="w4a8", router="matmul", router_scale=1.0 / 64.0),
    "skewed": LayerConfig("skewed", T=2048, H=4096, I=2048, E=256, k=6, x_dtype="bf16",
                          weight_format="w4a8", router="gumbel_zipf", router_scale=0.0,
                          zipf_s=1.1, n_shared=2),
    "fp8row": LayerConfig("fp8row", T=2048, H=4096, I=2048, E=384, k=6, x_dtype="bf16",
                          weight_format="fp8row", router="matmul", router_scale=1.0 / 64.0),
    # the NVFP4 + AQLM hybrid card's layer: hidden 6144, 256 experts of width 3072
    # (w13 [6144, 6144], w2 [6144, 3072]), 6 active, 14.8% of the experts hot
    "hybrid_decode": LayerConfig("hybrid_decode", T=4, H=6144, I=3072, E=256, k=6, x_dtype="bf16",
                                 weight_format="hybrid", router="gaussian", router_scale=0.0),
    "hybrid_tiny": LayerConfig("hybrid_tiny", T=16, H=256, I=128, E=8, k=2, x_dtype="f32",
                               weight_format="hybrid", router="gaussian", router_scale=0.0,
                               x_scale=1.0 / 16.0),
}
HYBRID_HOT_FRACTION = 0.148     # hot (NVFP4) share of the routed experts
# AQLM books: w13 one 65536-entry book; w2 a 65536-entry and a 256-entry book
AQLM_BOOKS = {"w13": (65536,), "w2": (65536, 256)}


def get_config(name: str, **overrides) -> LayerConfig:
    return dataclasses.replace(CONFIGS[name], **overrides)


# tensor ids used to key the generators
_TID = {"x": 1, "router": 2, "logits": 3, "w13": 4, "w2": 5, "zipf_rank": 6,
        "shared13": 7, "shared2": 8, "hybrid": 9, "nvfp4": 10, "aqlm": 11}


def tensor_seed(seed: int, tensor: str, index: int = 0) -> int:
    """A 63-bit generator seed for (seed, tensor, index)."""
    ss = np.random.SeedSequence([int(seed), _TID[tensor], int(index)])
    return int(ss.generate_state(2, dtype=np.uint32)[0]) | (
        int(ss.generate_state(2, dtype=np.uint32)[1] & 0x7FFFFFFF) << 32)


def _gen(device, seed: int, tensor: str, index: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, tensor, index))
    return g


def make_activations(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    """x: [T, H], fp32 (tiny) or bf16 (the Inkling-shaped layers)."""
    g = _gen(device, cfg.seed, "x")
    x = torch.randn(cfg.T, cfg.H, generator=g, device=device, dtype=torch.float32)
    x = x * cfg.x_scale
    return x.to(torch.bfloat16) if cfg.x_dtype == "bf16" else x


def router_weights(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    """The router matrix Wr [E, H] fp32 of a "matmul" router workload."""
    g = _gen(device, cfg.seed, "router")
    wr = torch.randn(cfg.E, cfg.H, generator=g, device=device, dtype=torch.float32)
    return wr * cfg.router_scale


def make_router(cfg: LayerConfig, x: torch.Tensor) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Router logits [T, E] fp32 and an optional per-expert bias [E] fp32.

    The router projection that produces the logits is the step *before* the
    expert layer; it is done here, once (torch fp32 matmul), so both sides
    receive identical logits.  Tests of the library's own router projection
    (moe_router_logits) take router_weights instead.
    """
    device = x.device
    if cfg.router == "matmul":
        wr = router_weights(cfg, device)
        logits = torch.matmul(x.to(torch.float32), wr.t()).contiguous()
        return logits, None
    if cfg.router == "gaussian":
        g = _gen(device, cfg.seed, "logits")
        return torch.randn(cfg.T, cfg.E, generator=g, device=device, dtype=torch.float32), None
    if cfg.router == "gumbel_zipf":
        # Top-1 popularity Zipf(s) over a seeded random ranking of the experts:
        # bias_e = -s * ln(rank_e) plus i.i.d. Gumbel(0,1) noise per (token, expert).
        g = _gen(device, cfg.seed, "logits")
        u = torch.rand(cfg.T, cfg.E, generator=g, device=device, dtype=torch.float64)
        u = u.clamp_min(1e-300)
        gumbel = (-torch.log(-torch.log(u))).to(torch.float32)
        gr = torch.Generator(device="cpu")
        gr.manual_seed(tensor_seed(cfg.seed, "zipf_rank"))
        rank = torch.randperm(cfg.E, generator=gr).to(torch.float64) + 1.0
        bias = (-cfg.zipf_s * torch.log(rank)).to(torch.float32).to(device)
        return gumbel.contiguous(), bias
    raise ValueError(cfg.router)


def expert_weight(cfg: LayerConfig, which: str, e: int, device="cpu") -> torch.Tensor:
    """Full-precision fp32 weight of one expert: w13 [2I, H] or w2 [H, I]."""
    shape = (2 * cfg.I, cfg.H) if which == "w13" else (cfg.H, cfg.I)
    g = _gen(device, cfg.seed, which, e)
    w = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return w * cfg.w_std


def iter_expert_weights(cfg: LayerConfig, which: str, device="cpu",
                        chunk: int = 16) -> Iterator[Tuple[int, torch.Tensor]]:
    """Yield (first expert, fp32 [n, N, K]) chunks of consecutive experts."""
    for e0 in range(0, cfg.E, chunk):
        n = min(chunk, cfg.E - e0)
        yield e0, torch.stack([expert_weight(cfg, which, e0 + i, device) for i in range(n)])


def make_shared_weights(cfg: LayerConfig, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 shared-expert weights, the n_shared experts fused into one MLP.

    Returns ws13 [2*S, H] (gate rows of every shared expert, then their up rows,
    S = n_shared * I) and ws2 [H, S] (their down projections side by side).
    Concatenating along the intermediate axis is an exact identity with summing
    the n_shared separate MLP outputs.
    """
    S = cfg.n_shared * cfg.I
    gates, ups, downs = [], [], []
    for j in range(cfg.n_shared):
        g = _gen(device, cfg.seed, "shared13", j)
        w = torch.randn(2 * cfg.I, cfg.H, generator=g, device=device) * cfg.w_std
        gates.append(w[: cfg.I])
        ups.append(w[cfg.I:])
        g = _gen(device, cfg.seed, "shared2", j)
        downs.append(torch.randn(cfg.H, cfg.I, generator=g, device=device) * cfg.w_std)
    ws13 = torch.cat(gates + ups, dim=0).to(torch.bfloat16).contiguous()
    ws2 = torch.cat(downs, dim=1).to(torch.bfloat16).contiguous()
    assert ws13.shape == (2 * S, cfg.H) and ws2.shape == (cfg.H, S)
    return ws13, ws2


def make_layer_inputs(cfg: LayerConfig, device="cpu", weights: bool = True) -> dict:
    """Everything one layer invocation needs (weights only for small configs)."""
    x = make_activations(cfg, device)
    logits, bias = make_router(cfg, x)
    out = {"x": x, "logits": logits, "bias": bias}
    if weights:
        out["w13"] = torch.stack([expert_weight(cfg, "w13", e, device) for e in range(cfg.E)])
        out["w2"] = torch.stack([expert_weight(cfg, "w2", e, device) for e in range(cfg.E)])
        if cfg.n_shared:
            out["ws13"], out["ws2"] = make_shared_weights(cfg, device)
    return out


def expected_distinct_experts(E: int, T: int, k: int) -> float:
    """E[#distinct experts] for T tokens each picking k of E uniformly (context only)."""
    return E * (1.0 - ((E - k) / E) ** T)


# ----------------------------------------------------------- hybrid experts
def hybrid_partition(cfg: LayerConfig) -> Tuple[np.ndarray, np.ndarray]:
    """(hot_ids, cold_ids): a seeded split of the experts, HYBRID_HOT_FRACTION hot."""
    rng = np.random.default_rng(tensor_seed(cfg.seed, "hybrid"))
    n_hot = max(1, int(round(HYBRID_HOT_FRACTION * cfg.E)))
    perm = rng.permutation(cfg.E)
    return np.sort(perm[:n_hot]).astype(np.int32), np.sort(perm[n_hot:]).astype(np.int32)


def make_nvfp4_slabs(cfg: LayerConfig, n_hot: int, device="cpu") -> dict:
    """Random NVFP4 slabs: uniform E2M1 code pairs, E4M3 block scales drawn from
    the bytes 0x30 .. 0x3F (0.5 .. 0.94), and per-slab scale2 around w_std / 4 (so
    the weights have roughly the spread of the other workloads)."""
    g = _gen(device, cfg.seed, "nvfp4")
    out = {}
    for proj, (n, k) in (("w13", (2 * cfg.I, cfg.H)), ("w2", (cfg.H, cfg.I))):
        out[proj] = torch.randint(0, 256, (n_hot, n, k // 2), generator=g, device=device,
                                  dtype=torch.uint8)
        out[proj + "_bs"] = torch.randint(0x30, 0x40, (n_hot, n, k // 16), generator=g,
                                          device=device, dtype=torch.uint8)
        out[proj + "_s2"] = (torch.rand(n_hot, generator=g, device=device) * 0.5 + 0.75) * (
            cfg.w_std / 4)
    return out


def make_aqlm_slabs(cfg: LayerConfig, n_cold: int, device="cpu") -> dict:
    """Random AQLM slabs: uniform codes over each book (int16 wraps above 32767),
    fp16 codebooks ~ N(0, w_std), fp16 row scales in [0.5, 1.5)."""
    g = _gen(device, cfg.seed, "aqlm")
    out = {}
    for proj, (n, k) in (("w13", (2 * cfg.I, cfg.H)), ("w2", (cfg.H, cfg.I))):
        codes, books = [], []
        for entries in AQLM_BOOKS[proj]:
            books.append((torch.randn(entries, 8, generator=g, device=device) * cfg.w_std).to(
                torch.float16))
            c = torch.randint(0, entries, (n_cold, n, k // 8), generator=g, device=device,
                              dtype=torch.int32)
            if entries > 256:
                codes.append(torch.where(c >= 32768, c - 65536, c).to(torch.int16))
            else:
                codes.append(c.to(torch.uint8))
        out[proj + "_codes"] = codes
        out[proj + "_books"] = books
        out[proj + "_scale"] = (torch.rand(n_cold, n, generator=g, device=device) + 0.5).to(
            torch.float16)
    return out
