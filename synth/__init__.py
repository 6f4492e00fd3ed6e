"""Seeded synthetic inputs for the MoE layer, shared by the GPU path's tests and
benchmark and by the oracle.

This module holds no arithmetic of the layer itself: it only describes the
workloads (shapes, routing options) and draws their random tensors. Each tensor
has a fixed id and its own ``torch.Generator`` seeded from (seed, id), so a
tensor never depends on which other tensors were drawn. Tensors are drawn on the
device they will be used on; the oracle always receives a copy of exactly the
bytes the GPU used.

Workloads follow the Switch explainer ("Mixture of Experts (MoE) を1から解説 —
Switch Transformerのルーティングと負荷分散", ta-paperlens.web.app: router, capacity
factor, aux loss, fp32 router, 0.1x init) and the shapes of the fine-grained
layers named on the "Mixture-of-Experts" concept page (notes.yuuk.io).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch

# tensor ids
TID_X, TID_WR, TID_W1, TID_W2, TID_BIAS, TID_DY, TID_SHARED, TID_NOISE = 1, 2, 3, 4, 5, 6, 7, 8


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                 # tokens in the batch
    d: int                 # d_model
    f: int                 # expert hidden width (per half for SwiGLU)
    E: int                 # routed experts
    k: int                 # experts per token
    gate: str = "softmax"  # "softmax" | "sigmoid_bias" | "sqrt_softplus_bias" | "noisy_topk"
    renorm: bool = False   # renormalise the k selected weights
    act: str = "relu"      # "relu" | "swiglu"
    dtype: str = "bf16"    # activations / expert weights: "bf16" | "f32"
    cf: float = 1.0        # capacity factor; <= 0 means no capacity limit
    alpha: float = 0.0     # aux-loss coefficient; 0 means no aux loss
    shared: int = 0        # number of always-on shared experts (0 or 1)
    logit_offset: str = "none"   # "none" | "normal" | "logzipf"
    sel_bias: str = "none"       # "none" | "uniform"
    router_init: str = "normal_fanin"  # "normal_fanin" | "truncnormal_small"
    fwd_only: bool = False
    routing: str = "token_choice"  # "token_choice" | "expert_choice" (then k = E)

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads. The first is the tiny fp32 case; the second is the
# Switch-Base-shaped layer the headline throughput is quoted on.
CONFIGS = {
    "tiny_f32": LayerConfig("tiny_f32", T=256, d=64, f=256, E=4, k=1, dtype="f32", cf=1.0,
                            router_init="truncnormal_small", fwd_only=True),
    "switch_base": LayerConfig("switch_base", T=8192, d=768, f=3072, E=128, k=1, cf=1.25,
                               alpha=0.01),
    "gshard_top2": LayerConfig("gshard_top2", T=16384, d=1024, f=4096, E=64, k=2, renorm=True,
                               cf=2.0, alpha=0.01, logit_offset="normal"),
    "finegrained_top8": LayerConfig("finegrained_top8", T=32768, d=2048, f=768, E=128, k=8,
                                    renorm=True, act="swiglu", cf=0.0, alpha=0.01,
                                    logit_offset="logzipf"),
    "deepseek_v3": LayerConfig("deepseek_v3", T=16384, d=7168, f=2048, E=256, k=8,
                               gate="sigmoid_bias", renorm=True, act="swiglu", cf=0.0,
                               shared=1, sel_bias="uniform"),
}
ORDER = ["tiny_f32", "switch_base", "gshard_top2", "finegrained_top8", "deepseek_v3"]

# Reduced versions with the same routing structure, small enough for the oracle to
# compute every output in seconds while still spanning several GEMM tiles and a
# ragged tail (T, d and f are deliberately not multiples of the tile sizes).
SMALL = {
    "tiny_f32": CONFIGS["tiny_f32"],
    "switch_base": CONFIGS["switch_base"].replace(name="switch_base_s", T=1000, d=256, f=384, E=16),
    "gshard_top2": CONFIGS["gshard_top2"].replace(name="gshard_top2_s", T=777, d=192, f=320, E=8),
    "finegrained_top8": CONFIGS["finegrained_top8"].replace(name="finegrained_top8_s", T=600, d=256,
                                                            f=136, E=16, k=4),
    "deepseek_v3": CONFIGS["deepseek_v3"].replace(name="deepseek_v3_s", T=300, d=320, f=200, E=32,
                                                  k=4),
}


def _gen(seed: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + tid)
    return g


def _normal(shape, std, g, device, chunks=1):
    """N(0, std^2) in fp32, drawn in ``chunks`` pieces along dim 0 (bounded memory)."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    n0 = shape[0]
    step = max(1, math.ceil(n0 / chunks))
    for a in range(0, n0, step):
        b = min(n0, a + step)
        out[a:b] = torch.randn((b - a,) + tuple(shape[1:]), generator=g, device=device) * std
    return out


def _truncnormal(shape, std, g, device):
    """N(0, std^2) truncated at +-2 std by redrawing the samples outside."""
    out = torch.randn(shape, generator=g, device=device)
    while True:
        bad = out.abs() > 2.0
        nb = int(bad.sum())
        if nb == 0:
            break
        out[bad] = torch.randn(nb, generator=g, device=device)
    return out * std


def make_inputs(cfg: LayerConfig, seed: int = 0, device="cpu", with_dy: bool = True) -> dict:
    """Draw every input tensor of one layer call.

    x ~ N(0,1); expert weights ~ N(0, 1/fan_in); W_r ~ N(0, 1/d) (2E rows, clean and
    noise, for noisy top-k gating, whose noise eps ~ N(0,1) is drawn too) except the tiny
    workload's truncated N(0, (0.1/sqrt(d))^2) (the Switch 0.1x init scale);
    logit offsets ~ N(0,1) ("normal") or -1.1*ln(e+1) ("logzipf", Zipf s=1.1
    popularity with expert 0 the most popular); selection bias ~ U(-0.5, 0.5);
    upstream gradient dy ~ N(0,1). Activations and expert weights are rounded
    to the workload's storage dtype (round to nearest even for bf16); router
    tensors stay fp32.
    """
    dev = torch.device(device)
    act_dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    T, d, f, E = cfg.T, cfg.d, cfg.f, cfg.E
    f1 = 2 * f if cfg.act == "swiglu" else f
    big = dev.type != "cpu"
    out = {}
    out["x"] = _normal((T, d), 1.0, _gen(seed, TID_X, dev), dev).to(act_dt)
    ER = 2 * E if cfg.gate == "noisy_topk" else E  # noisy gating stacks [W_g; W_noise]
    if cfg.router_init == "truncnormal_small":
        out["w_router"] = _truncnormal((ER, d), 0.1 / math.sqrt(d), _gen(seed, TID_WR, dev), dev)
    else:
        out["w_router"] = _normal((ER, d), 1.0 / math.sqrt(d), _gen(seed, TID_WR, dev), dev)
    if cfg.gate == "noisy_topk":
        out["noise"] = _normal((T, E), 1.0, _gen(seed, TID_NOISE, dev), dev)
    g1 = _gen(seed, TID_W1, dev)
    g2 = _gen(seed, TID_W2, dev)
    w1 = torch.empty((E, f1, d), dtype=act_dt, device=dev)
    w2 = torch.empty((E, d, f), dtype=act_dt, device=dev)
    for e in range(E):  # one expert at a time keeps the fp32 staging small
        w1[e] = _normal((f1, d), 1.0 / math.sqrt(d), g1, dev).to(act_dt)
        w2[e] = _normal((d, f), 1.0 / math.sqrt(f), g2, dev).to(act_dt)
    out["w1"], out["w2"] = w1, w2
    gb = _gen(seed, TID_BIAS, dev)
    if cfg.logit_offset == "normal":
        out["logit_offset"] = torch.randn(E, generator=gb, device=dev)
    elif cfg.logit_offset == "logzipf":
        out["logit_offset"] = (-1.1 * torch.log(torch.arange(1, E + 1, dtype=torch.float64))).to(
            torch.float32).to(dev)
    if cfg.sel_bias == "uniform":
        out["sel_bias"] = torch.rand(E, generator=gb, device=dev) - 0.5
    if cfg.shared:
        gs = _gen(seed, TID_SHARED, dev)
        out["ws1"] = _normal((f1, d), 1.0 / math.sqrt(d), gs, dev, chunks=8 if big else 1).to(act_dt)
        out["ws2"] = _normal((d, f), 1.0 / math.sqrt(f), gs, dev, chunks=8 if big else 1).to(act_dt)
    if with_dy and not cfg.fwd_only:
        out["dy"] = _normal((T, d), 1.0, _gen(seed, TID_DY, dev), dev).to(act_dt)
    return out
