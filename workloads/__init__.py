"""Seeded synthetic inputs for the NVFP4 expert layer.

This module only draws inputs; it holds none of the layer's arithmetic (no
quantization, no GEMM, no SiLU). Tests, the oracle side and the GPU side all
take their inputs from here, so both sides see identical bits.

Everything is drawn on the CPU with torch's seeded generator (its output does
not depend on the thread count or the device) and returned as NumPy arrays:
bf16 values as uint16 bit patterns, routing ids as int32, routing weights as
float32. Weights are drawn in bf16; turning them into NVFP4 is the quantizer's
job (oracle side: oracle.quantize; GPU side: nvfp4_quantize_weights).

Recipes (shapes from the pages' layer: hidden 7168, intermediate 3072, 48 local
experts, w13 (48, 3584, 6144) and w2 (48, 1536, 7168) packed bytes; magnitudes
from the pages' traces: activation amax about 5-10):

* x: bf16(N(0,1) * x_std); the prefill recipe sets 0.1% of positions, chosen
  uniformly, to +-40 with a random sign;
* weights: bf16(N(0, 0.02)), drawn expert by expert;
* routing: logits N(0,1) of shape (T, E), plus an optional per-expert bias; ids
  are the top-k logits (distinct experts), weights the softmax over the k
  selected logits (renormalized softmax), float32;
* skewed routing bias: 2.0 * ln(p_r) with p_r the Zipf(s=1.2) pmf over ranks
  1..E, ranks assigned to experts by a seeded permutation;
* skewed alphas: log-uniform in [1e-4, 1e-2].
"""
import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    topk: int
    seed_x: int
    seed_w: int
    x_std: float = 3.0
    outlier_frac: float = 0.0
    outlier_value: float = 40.0
    zipf_s: float = 0.0          # 0 = no skew bias
    zipf_bias_scale: float = 2.0
    alpha_loguniform: bool = False

    @property
    def slots(self):
        return self.T * self.topk


TINY = LayerConfig("tiny", T=32, H=256, I=128, E=4, topk=2, seed_x=1, seed_w=1)
DECODE = LayerConfig("decode", T=8, H=7168, I=3072, E=48, topk=8, seed_x=30, seed_w=3,
                     x_std=1.5)
PREFILL = LayerConfig("prefill", T=4096, H=7168, I=3072, E=48, topk=8, seed_x=40, seed_w=3,
                      outlier_frac=1e-3)
SKEWED = LayerConfig("skewed", T=8192, H=7168, I=3072, E=48, topk=8, seed_x=50, seed_w=3,
                     outlier_frac=1e-3, zipf_s=1.2, alpha_loguniform=True)
LAYER_CONFIGS = {c.name: c for c in (TINY, DECODE, PREFILL, SKEWED)}


@dataclass(frozen=True)
class GemmConfig:
    name: str
    M: int
    N: int
    K: int
    seed: int
    a_std: float = 3.0
    w_std: float = 0.02


DENSE = GemmConfig("dense", M=256, N=6144, K=7168, seed=2)

WEIGHT_STD = 0.02


def _gen(seed, stream):
    """Independent sub-stream `stream` of master seed `seed`."""
    g = torch.Generator()
    g.manual_seed(int(seed) * 1_000_003 + int(stream) * 7919 + 12345)
    return g


def bf16_bits_from_tensor(t):
    """float32 torch tensor -> bf16 bit patterns (torch's nearest-even cast)."""
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, std, seed, stream):
    g = _gen(seed, stream)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32) * float(std)
    return bf16_bits_from_tensor(t)


def activations(cfg: LayerConfig):
    """x (T, H) as bf16 bits."""
    g = _gen(cfg.seed_x, 1)
    t = torch.randn((cfg.T, cfg.H), generator=g, dtype=torch.float32) * float(cfg.x_std)
    if cfg.outlier_frac > 0:
        n = cfg.T * cfg.H
        n_out = max(1, int(round(cfg.outlier_frac * n)))
        pos = torch.randperm(n, generator=g)[:n_out]
        sign = torch.where(torch.rand(n_out, generator=g) < 0.5, -1.0, 1.0)
        t.view(-1)[pos] = sign * float(cfg.outlier_value)
    return bf16_bits_from_tensor(t)


def expert_weights_bf16(cfg: LayerConfig, e: int):
    """(w13 (H, 2I) = [gate | up] along N, w2 (I, H)) of expert e, bf16 bits.

    Stored as the math layout W (K, N): y = x @ W.
    """
    w13 = normal_bf16((cfg.H, 2 * cfg.I), WEIGHT_STD, cfg.seed_w, 1000 + 2 * e)
    w2 = normal_bf16((cfg.I, cfg.H), WEIGHT_STD, cfg.seed_w, 1001 + 2 * e)
    return w13, w2


def zipf_bias(cfg: LayerConfig):
    if cfg.zipf_s <= 0:
        return np.zeros(cfg.E, dtype=np.float32)
    ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
    p = ranks ** (-cfg.zipf_s)
    p /= p.sum()
    bias_by_rank = cfg.zipf_bias_scale * np.log(p)
    g = _gen(cfg.seed_x, 3)
    perm = torch.randperm(cfg.E, generator=g).numpy()
    bias = np.empty(cfg.E, dtype=np.float64)
    bias[perm] = bias_by_rank          # expert perm[r] gets rank r+1
    return bias.astype(np.float32)


def routing(cfg: LayerConfig):
    """(topk_ids int32 (T, k), topk_weights float32 (T, k))."""
    g = _gen(cfg.seed_x, 2)
    logits = torch.randn((cfg.T, cfg.E), generator=g, dtype=torch.float64)
    logits = logits + torch.from_numpy(zipf_bias(cfg).astype(np.float64))[None, :]
    vals, ids = torch.topk(logits, cfg.topk, dim=1)
    w = torch.softmax(vals, dim=1)
    return ids.to(torch.int32).numpy(), w.to(torch.float32).numpy()


def alphas_loguniform(cfg: LayerConfig):
    """(w13_alpha, w2_alpha) float32 (E,), independent log-uniform [1e-4, 1e-2]."""
    g = _gen(cfg.seed_w, 4)
    u = torch.rand((2, cfg.E), generator=g, dtype=torch.float64)
    a = torch.exp(math.log(1e-4) + u * (math.log(1e-2) - math.log(1e-4)))
    a = a.to(torch.float32).numpy()
    return a[0].copy(), a[1].copy()


def dense_gemm_inputs(cfg: GemmConfig = DENSE):
    """(A (M, K) bf16 bits, B (K, N) bf16 bits)."""
    a = normal_bf16((cfg.M, cfg.K), cfg.a_std, cfg.seed, 1)
    b = normal_bf16((cfg.K, cfg.N), cfg.w_std, cfg.seed, 2)
    return a, b


def small_layer(name, T, H, I, E, topk, seed, x_std=3.0, zipf_s=0.0,
                alpha_loguniform=False, outlier_frac=0.0):
    """A layer config of arbitrary (small) shape for parity sweeps."""
    return LayerConfig(name, T=T, H=H, I=I, E=E, topk=topk, seed_x=seed,
                       seed_w=seed + 100, x_std=x_std, zipf_s=zipf_s,
                       alpha_loguniform=alpha_loguniform, outlier_frac=outlier_frac)
