"""Seeded synthetic inputs for the MoE feed-forward layer.

Shared by the tests, the smoke check and the benchmark, for both the GPU
library and the CPU oracle.  It draws tensors of the workloads' shapes and
distributions and converts them for the oracle; it holds none of the layer's
arithmetic.

Workloads (d=4096, f=14336, E=8, k=2 are the layer shapes of the Mixtral of
Experts pages' hyperparameter table):
  tiny     fp32  T=64     d=128  f=256    x ~ N(0,1), seed 0 (CPU generator)
  decode   bf16  T=32     x ~ N(0,1), each row scaled to unit RMS (eps 1e-5)
  prefill  bf16  T=4096   as decode (one 4096-token sequence)
  skewed   bf16  T=16384  as decode, plus per-expert logit bias
                          (2, 1, .5, 0, 0, 0, -.5, -1)
  stack    bf16  T=2048   h0 ~ N(0,1); 32 layers of independent weights
Weights: w_router [d,E], w1/w3 [E,d,f], w2 [E,f,d], each entry ~ N(0, s^2)
with standard deviation s = 1/sqrt(fan_in) (fan_in = d for w_router, w1, w3
and f for w2), drawn in fp32 and rounded to nearest-even bf16 for the bf16
workloads.  Public benchmark text is not available; these tensors stand in for
hidden states with unit RMS and near-uniform routing.
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16"
    T: int
    d: int
    f: int
    E: int
    k: int
    x_dist: str         # "normal" or "rms" (rows scaled to unit RMS)
    bias: tuple | None = None
    layers: int = 1
    rms_eps: float = 1e-5

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


SKEW_BIAS = (2.0, 1.0, 0.5, 0.0, 0.0, 0.0, -0.5, -1.0)

WORKLOADS = {
    "tiny": Workload("tiny", "f32", 64, 128, 256, 8, 2, "normal"),
    "decode": Workload("decode", "bf16", 32, 4096, 14336, 8, 2, "rms"),
    "prefill": Workload("prefill", "bf16", 4096, 4096, 14336, 8, 2, "rms"),
    "skewed": Workload("skewed", "bf16", 16384, 4096, 14336, 8, 2, "rms", SKEW_BIAS),
    "stack": Workload("stack", "bf16", 2048, 4096, 14336, 8, 2, "normal", None, 32),
}


def tensor_seed(seed: int, workload: str, layer: int, tensor: str) -> int:
    """Stable 31-bit seed for one tensor of one layer of one workload."""
    key = "%d/%s/%d/%s" % (seed, workload, layer, tensor)
    return zlib.crc32(key.encode()) & 0x7FFFFFFF


def _normal(shape, std, seed, device, out_dtype, chunk_dim0=True):
    """N(0, std^2) in fp32, rounded (RNE) to out_dtype; drawn per leading slice."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=out_dtype, device=device)
    if chunk_dim0 and len(shape) == 3:
        for i in range(shape[0]):
            z = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
            out[i].copy_(z.mul_(std))
    else:
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.copy_(z.mul_(std))
    return out


def make_router(d, E, dtype, device, seed=0, workload="case", layer=0):
    """w_router [d,E] with std 1/sqrt(d)."""
    s_d = 1.0 / float(np.sqrt(d))
    return _normal((d, E), s_d, tensor_seed(seed, workload, layer, "w_router"), device, dtype)


def make_experts(d, f, E, dtype, device, seed=0, workload="case", layer=0):
    """w1 [E,d,f], w3 [E,d,f] with std 1/sqrt(d); w2 [E,f,d] with std 1/sqrt(f)."""
    s_d = 1.0 / float(np.sqrt(d))
    s_f = 1.0 / float(np.sqrt(f))
    return {
        "w1": _normal((E, d, f), s_d, tensor_seed(seed, workload, layer, "w1"), device, dtype),
        "w3": _normal((E, d, f), s_d, tensor_seed(seed, workload, layer, "w3"), device, dtype),
        "w2": _normal((E, f, d), s_f, tensor_seed(seed, workload, layer, "w2"), device, dtype),
    }


def make_weights(d, f, E, dtype, device, seed=0, workload="case", layer=0):
    """All four weight tensors of one layer."""
    res = {"w_router": make_router(d, E, dtype, device, seed, workload, layer)}
    res.update(make_experts(d, f, E, dtype, device, seed, workload, layer))
    return res


def make_x(T, d, dtype, device, x_dist="normal", seed=0, workload="case", rms_eps=1e-5):
    """Activations [T,d]: N(0,1), optionally each row scaled to unit RMS in fp32."""
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, workload, 0, "x"))
    z = torch.randn((T, d), generator=g, device=device, dtype=torch.float32)
    if x_dist not in ("normal", "rms"):
        raise ValueError(x_dist)
    if x_dist == "rms" and T > 0:
        z = z * torch.rsqrt(z.pow(2).mean(dim=1, keepdim=True) + rms_eps)
    return z.to(dtype)


def tiny_inputs():
    """The tiny fp32 workload: CPU generator seeded 0, drawn in the order
    x, w_router, w1, w3, w2."""
    wl = WORKLOADS["tiny"]
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    T, d, f, E = wl.T, wl.d, wl.f, wl.E
    x = torch.randn((T, d), generator=g)
    wr = torch.randn((d, E), generator=g) / np.sqrt(d)
    w1 = torch.randn((E, d, f), generator=g) / np.sqrt(d)
    w3 = torch.randn((E, d, f), generator=g) / np.sqrt(d)
    w2 = torch.randn((E, f, d), generator=g) / np.sqrt(f)
    return {"x": x, "w_router": wr.float(), "w1": w1.float(), "w3": w3.float(), "w2": w2.float()}


def workload_inputs(name, device, seed=0, layer=0, with_x=True):
    """Inputs of a named workload (one layer for 'stack'); tensors on ``device``."""
    wl = WORKLOADS[name]
    if name == "tiny":
        t = tiny_inputs()
        res = {kk: v.to(device) for kk, v in t.items()}
    else:
        res = make_weights(wl.d, wl.f, wl.E, wl.torch_dtype, device, seed, name, layer)
        if with_x:
            res["x"] = make_x(wl.T, wl.d, wl.torch_dtype, device, wl.x_dist, seed, name, wl.rms_eps)
    res["bias"] = None if wl.bias is None else torch.tensor(wl.bias, dtype=torch.float32, device=device)
    return res


def host_array(t: torch.Tensor) -> np.ndarray:
    """A tensor as a host numpy array the oracle accepts: float32 stays
    float32; bfloat16 becomes its uint16 bit patterns (no rounding)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float64 exactly."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
