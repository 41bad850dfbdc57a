"""Seeded synthetic inputs and workload shapes for the Summaryformer memory.

This module is the only thing the HIP path's tests and the oracle share.  It
draws random tensors and names workload shapes; it holds none of the memory's
arithmetic (no slot map, no eviction, no attention).

Every Q, K and V tensor is i.i.d. N(0, 1), drawn in float32 by
``torch.randn`` from a generator seeded with a 64-bit key that names the
tensor, then (for the long-horizon workload) V is multiplied by 0.5, then the
tensor is cast to the workload's storage type with round-to-nearest-even.
The oracle always receives host copies of the very bytes the GPU receives.

Shapes follow the model card "GTA world model: weights and inference code":
the served grid (24x42 = 1008 raw tokens, X = 96 summary tokens, Y = 2,
W = 24, from its parameter table under "One buffer, no mask") and scaled
variants of it.  The page trains on its own video dataset; no dataset is used
here, synthetic tensors of the same shapes stand in for the per-block Q/K/V.
"""
from __future__ import annotations

import torch

Q, K, V = 0, 1, 2
BIAS = 3  # a recency bias table (one per session)

# name -> shape and seed of each workload.  Keys mirror the C-ABI's sf_config
# fields; "frames" lists the frame ids a workload steps through (or, for the
# batched one, the fill level of each session).
WORKLOADS = {
    # 1 block, 1 head of 64, 4x6 grid + 4 summaries, Y=2, W=6, 12 frames.
    "tiny": dict(hw=24, x=4, y=2, w=6, n_heads=1, head_dim=64, n_blocks=1,
                 dtype="f32", frames=list(range(12)), seed=0, v_scale=1.0),
    # served grid, one block, the buffer as it stands at frame 31.
    "served1": dict(hw=1008, x=96, y=2, w=24, n_heads=16, head_dim=64,
                    n_blocks=1, dtype="bf16", frames=list(range(32)), seed=1,
                    v_scale=1.0),
    # the server's default window (W = 16), served grid, two blocks, 40 frames.
    "served16": dict(hw=1008, x=96, y=2, w=16, n_heads=16, head_dim=64,
                     n_blocks=2, dtype="bf16", frames=list(range(40)), seed=5, v_scale=1.0),
    # served grid through 28 blocks for 64 frames.
    "rollout": dict(hw=1008, x=96, y=2, w=24, n_heads=16, head_dim=64,
                    n_blocks=28, dtype="bf16", frames=list(range(64)), seed=2,
                    v_scale=1.0),
    # 8 independent sessions at different fill levels, 28 blocks.
    "batched": dict(hw=1008, x=96, y=2, w=24, n_heads=16, head_dim=64,
                    n_blocks=28, dtype="bf16", frames=[0, 1, 2, 3, 10, 23, 24, 31],
                    seed=3, v_scale=1.0),
    # long horizon: 45x80 grid + 256 summaries, Y=4, W=96, 24 heads of 128.
    "long": dict(hw=3600, x=256, y=4, w=96, n_heads=24, head_dim=128,
                 n_blocks=28, dtype="bf16", frames=list(range(128)), seed=4,
                 v_scale=0.5),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def tensor_key(seed: int, session: int, block: int, t: int, which: int) -> int:
    """64-bit generator seed naming one tensor (seed, session, block, frame, Q/K/V)."""
    if not (0 <= session < 256 and 0 <= block < 256 and 0 <= t < (1 << 20) and which in (Q, K, V, BIAS)):
        raise ValueError("tensor_key: field out of range")
    return ((((seed * 256 + session) * 256 + block) << 20 | t) << 4) | which


def draw(shape, key: int, dtype: str, device="cpu", scale: float = 1.0) -> torch.Tensor:
    """One N(0,1) float32 tensor from generator ``key``, times ``scale``, cast to ``dtype``."""
    g = torch.Generator(device=device)
    g.manual_seed(key)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(TORCH_DTYPE[dtype])


def record_shape(wl: dict):
    """[rows of one record][heads][head_dim] for a workload dict."""
    return (wl["hw"] + wl["x"], wl["n_heads"], wl["head_dim"])


def frame_tensors(wl: dict, session: int, block: int, t: int, device="cpu"):
    """(q, k, v) of one block at frame t, each [R][H][d] in the workload dtype."""
    shp = record_shape(wl)
    seed, dt = wl["seed"], wl["dtype"]
    q = draw(shp, tensor_key(seed, session, block, t, Q), dt, device)
    k = draw(shp, tensor_key(seed, session, block, t, K), dt, device)
    v = draw(shp, tensor_key(seed, session, block, t, V), dt, device, wl.get("v_scale", 1.0))
    return q, k, v


def bias_table(wl: dict, session: int, version: int = 0, scale: float = 2.0, device="cpu") -> torch.Tensor:
    """A recency bias table [n_heads][w + 1] in float32: i.i.d. N(0, 1) times ``scale``,
    drawn from the generator of (seed, session, block 0, frame ``version``, BIAS)."""
    return draw((wl["n_heads"], wl["w"] + 1), tensor_key(wl["seed"], session, 0, version, BIAS), "f32", device, scale)


def to_host_bytes(x: torch.Tensor):
    """Host numpy copy of a tensor's bytes: uint16 bit patterns for bf16, float32 otherwise."""
    import numpy as np
    x = x.detach().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()
