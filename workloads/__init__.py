"""Seeded synthetic inputs for the fused GEMM + epilogue workloads.

This module only draws random numbers and lays them out; it holds none of the
operations the library computes, so both the HIP path's callers and the CPU oracle's
callers can take inputs from it without sharing any arithmetic.

Recipe: every tensor comes from its own torch.Generator seeded with 1000*cfg + t
(t = 1 X/x, 2 W/Wg, 3 bias/Wu, 4 dY/Wd, 5 P/dout), drawn as float32 standard normals,
scaled in float32 and then rounded to the workload's half type.  The sizes and scales
follow the pages' workloads: the H200 fp16 linear-layer shape (65536 x 16384) x
(16384 x 8192) of "Fusing Matmul Epilogs with nvmath-python" ("Suitable evaluation
scenarios"), and the bf16 SwiGLU-MLP shape H=5120, I=17408 with 0.02-scaled weights of
gemm_swiglu_mlp_fusion.py (_demo).
"""
from dataclasses import dataclass

import numpy as np
import torch


def seed_of(cfg, t):
    return 1000 * cfg + t


def randn(shape, seed, scale=1.0, dtype=torch.float16, device="cpu"):
    """Seeded N(0, scale^2) tensor: float32 normals, scaled in float32, then rounded."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def random_mask_words(m, n, seed, ld_aux=None, device="cpu"):
    """relu_aux words whose first n bits per row are independent fair coin flips.

    This is the distribution of the packed signs of an independent N(0,1)
    pre-activation (each element is positive with probability 1/2).  Bits past column
    n-1 and padding words past ceil(n/32) are zero.  Returned as int32 (the bit
    pattern of the uint32 words).
    """
    nw = (n + 31) // 32
    ld_aux = nw if ld_aux is None else ld_aux
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randint(-(2 ** 31), 2 ** 31, (m, nw), generator=g, dtype=torch.int64, device=device)
    if n % 32:
        w[:, nw - 1] &= (1 << (n % 32)) - 1
    out = torch.zeros((m, ld_aux), dtype=torch.int32, device=device)
    out[:, :nw] = w.to(torch.int32)
    return out


def to_numpy(t):
    """Host numpy copy.  fp16 stays float16; bf16 becomes its uint16 bit patterns;
    int32 mask words become uint32."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


@dataclass(frozen=True)
class LinearCfg:
    """A ReLU linear layer: X (m x k) . W (k x n) + bias; backward dY (m x n) . W^T."""
    cfg: int
    m: int
    n: int
    k: int
    w_scale: float
    bias_scale: float
    mask_from: str  # "forward" (square layer, reuse the forward mask) or "separate"


@dataclass(frozen=True)
class SwigluCfg:
    """SwiGLU MLP: x (m x h), Wg/Wu (i x h), Wd (h x i), all scaled 0.02."""
    cfg: int
    m: int
    h: int
    i: int
    w_scale: float = 0.02


LINEAR = {
    1: LinearCfg(1, 32, 64, 128, 1.0, 1.0, "separate"),
    2: LinearCfg(2, 4096, 4096, 4096, 1.0 / 64.0, 0.1, "forward"),
    3: LinearCfg(3, 65536, 8192, 16384, 1.0 / 128.0, 0.1, "separate"),
}
SWIGLU = {
    4: SwigluCfg(4, 2048, 5120, 17408),
    5: SwigluCfg(5, 16384, 5120, 17408),
}


def linear_inputs(c, device="cpu", m=None, n=None, k=None):
    """fp16 X, W (k x n), bias, dY and a separate relu_aux for the backward.

    The separate mask stands for the previous layer's relu_aux over an M x K
    pre-activation drawn N(0,1); for the square layer the forward's own mask is used
    instead by the caller.
    """
    m = c.m if m is None else m
    n = c.n if n is None else n
    k = c.k if k is None else k
    x = randn((m, k), seed_of(c.cfg, 1), 1.0, torch.float16, device)
    w = randn((k, n), seed_of(c.cfg, 2), c.w_scale, torch.float16, device)
    bias = randn((n,), seed_of(c.cfg, 3), c.bias_scale, torch.float16, device)
    dy = randn((m, n), seed_of(c.cfg, 4), 1.0, torch.float16, device)
    mask = random_mask_words(m, k, seed_of(c.cfg, 5), device=device)
    return {"x": x, "w": w, "bias": bias, "dy": dy, "mask_in": mask}


def swiglu_inputs(c, device="cpu", m=None, h=None, i=None):
    m = c.m if m is None else m
    h = c.h if h is None else h
    i = c.i if i is None else i
    x = randn((m, h), seed_of(c.cfg, 1), 1.0, torch.bfloat16, device)
    wg = randn((i, h), seed_of(c.cfg, 2), c.w_scale, torch.bfloat16, device)
    wu = randn((i, h), seed_of(c.cfg, 3), c.w_scale, torch.bfloat16, device)
    wd = randn((h, i), seed_of(c.cfg, 4), c.w_scale, torch.bfloat16, device)
    return {"x": x, "wg": wg, "wu": wu, "wd": wd}


def dswiglu_inputs(c, device="cpu", m=None, h=None, i=None):
    """dout, Wd and the saved bf16 gate/up pre-activations.

    gate and up are the bf16 results of x Wg^T and x Wu^T for a seeded x, as the
    SwiGLU forward would have saved them; they are produced with torch's own matmul
    (neither this library nor the oracle) purely as realistic input data.
    """
    m = c.m if m is None else m
    h = c.h if h is None else h
    i = c.i if i is None else i
    base = swiglu_inputs(c, device, m, h, i)
    dout = randn((m, h), seed_of(c.cfg, 5), 1.0, torch.bfloat16, device)
    gate = torch.matmul(base["x"], base["wg"].t().contiguous())
    up = torch.matmul(base["x"], base["wu"].t().contiguous())
    return {"dout": dout, "wd": base["wd"], "gate": gate, "up": up}
