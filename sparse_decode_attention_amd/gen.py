"""Seeded synthetic q/k/v for SparK workloads.

This module only draws random tensors; it holds none of the method's
arithmetic, and both the GPU path and the CPU oracle receive its output as
plain inputs.

Distribution (channel-heterogeneous, heavy-tailed, so that per-token channel
saliency varies strongly as the SparK walkthrough's section 1 and Fig. 1
describe): x = z * s_c * e_tc with z ~ N(0,1) per element, s_c ~ LogNormal(0,1)
per (tensor, layer, head, channel) and e_tc ~ LogNormal(0,1) per element.
x is formed in fp32 and rounded to bf16 (round to nearest even). The window
queries and the decode queries of a layer share the query tensor's s_c.

Two backends draw from this distribution:
- ``numpy``: NumPy ``default_rng(SeedSequence([seed, cfg, tensor, layer,
  stream, b, head]))``, one stream per (batch, head) slab, on the host;
- ``torch``: a seeded ``torch.Generator`` on the target device, for shapes too
  large to draw on the host (the 32-layer stack).
The backends give different values from the same distribution; a test always
feeds one backend's tensors to both sides.

bf16 tensors are carried as uint16 bit patterns on the host (NumPy has no
bf16) and as ``torch.bfloat16`` on the device.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload

T_Q, T_K, T_V = 0, 1, 2
_SCALE_STREAM = 1_000_000


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def channel_scales(seed: int, cfg: int, tensor: int, layer: int, n_heads: int, D: int) -> np.ndarray:
    """s_c ~ LogNormal(0,1), shape [n_heads][D], fp32."""
    r = _rng(seed, cfg, tensor, layer, _SCALE_STREAM)
    return np.exp(r.standard_normal((n_heads, D), dtype=np.float32))


def _slab(seed, cfg, tensor, layer, stream, b, h, rows, D, s_c):
    r = _rng(seed, cfg, tensor, layer, stream, b, h)
    z = r.standard_normal((rows, D), dtype=np.float32)
    e = np.exp(r.standard_normal((rows, D), dtype=np.float32))
    return f32_to_bf16_bits(z * s_c[None, :] * e)


def numpy_tensor(seed: int, cfg: int, tensor: int, layer: int, stream: int,
                 B: int, n_heads: int, rows: int, D: int) -> np.ndarray:
    """bf16 bits [B][n_heads][rows][D] drawn slab by slab (bounded host memory)."""
    s = channel_scales(seed, cfg, tensor, layer, n_heads, D)
    out = np.empty((B, n_heads, rows, D), dtype=np.uint16)
    for b in range(B):
        for h in range(n_heads):
            out[b, h] = _slab(seed, cfg, tensor, layer, stream, b, h, rows, D, s[h])
    return out


def numpy_layer(w: Workload, seed: int = 0, layer: int = 0, steps: int | None = None,
                S: int | None = None) -> dict:
    """Host inputs of one layer as bf16 bit arrays.

    q_win [B][n_q][W][D]  (the last W prompt queries)
    k, v  [B][n_kv][S][D]
    q_dec [steps][B][n_q][D]  (decode step s draws stream s+1)
    """
    S = w.S if S is None else S
    steps = w.steps if steps is None else steps
    q_win = numpy_tensor(seed, w.cfg_id, T_Q, layer, 0, w.B, w.n_q, w.window, w.D)
    k = numpy_tensor(seed, w.cfg_id, T_K, layer, 0, w.B, w.n_kv, S, w.D)
    v = numpy_tensor(seed, w.cfg_id, T_V, layer, 0, w.B, w.n_kv, S, w.D)
    q_dec = np.stack([numpy_tensor(seed, w.cfg_id, T_Q, layer, s + 1, w.B, w.n_q, 1, w.D)[:, :, 0, :]
                      for s in range(steps)]) if steps > 0 else np.zeros((0, w.B, w.n_q, w.D), np.uint16)
    return {"q_win": q_win, "k": k, "v": v, "q_dec": q_dec}


# ---------------------------------------------------------------- torch backend

def _torch_seed(*key: int) -> int:
    ss = np.random.SeedSequence([int(k) for k in key])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def torch_tensor(seed: int, cfg: int, tensor: int, layer: int, stream: int,
                 B: int, n_heads: int, rows: int, D: int, device, out=None):
    """bf16 tensor [B][n_heads][rows][D] drawn on ``device`` (chunked per batch row)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, cfg, tensor, layer, _SCALE_STREAM, 7))
    s_c = torch.exp(torch.randn((n_heads, 1, D), generator=g, device=device, dtype=torch.float32))
    if out is None:
        out = torch.empty((B, n_heads, rows, D), device=device, dtype=torch.bfloat16)
    g.manual_seed(_torch_seed(seed, cfg, tensor, layer, stream))
    for b in range(B):
        z = torch.randn((n_heads, rows, D), generator=g, device=device, dtype=torch.float32)
        e = torch.randn((n_heads, rows, D), generator=g, device=device, dtype=torch.float32).exp_()
        out[b].copy_((z.mul_(s_c).mul_(e)).to(torch.bfloat16))
        del z, e
    return out


def torch_layer(w: Workload, device, seed: int = 0, layer: int = 0, steps: int | None = None,
                S: int | None = None) -> dict:
    """Device inputs of one layer (torch.bfloat16), same shapes as ``numpy_layer``."""
    import torch
    S = w.S if S is None else S
    steps = w.steps if steps is None else steps
    q_win = torch_tensor(seed, w.cfg_id, T_Q, layer, 0, w.B, w.n_q, w.window, w.D, device)
    k = torch_tensor(seed, w.cfg_id, T_K, layer, 0, w.B, w.n_kv, S, w.D, device)
    v = torch_tensor(seed, w.cfg_id, T_V, layer, 0, w.B, w.n_kv, S, w.D, device)
    q_dec = torch.stack([torch_tensor(seed, w.cfg_id, T_Q, layer, s + 1, w.B, w.n_q, 1, w.D, device)[:, :, 0, :]
                         for s in range(steps)]) if steps > 0 else \
        torch.zeros((0, w.B, w.n_q, w.D), device=device, dtype=torch.bfloat16)
    return {"q_win": q_win, "k": k, "v": v, "q_dec": q_dec}


def to_torch_bf16(bits: np.ndarray, device=None):
    """Host bf16 bits -> torch.bfloat16 tensor (bit-for-bit)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t
