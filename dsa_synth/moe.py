"""Seeded synthetic inputs for the MoE expert product (MXFP4 weights, FP8
tokens, routing), shared by the oracle side and the GPU side of the parity
tests and by the benchmark.

Nothing here computes any part of the method: the module draws random
bytes and counts.  Token values are made with torch's own float ->
float8_e4m3fn cast (a library conversion).

Recipes:
  * weight codes: uniform random bytes (every FP4 code, both nibbles);
  * scales: E8M0 codes uniform on [scale_lo, scale_hi]; 126..128 (2^-1 ..
    2^1) keeps every product sum exact in fp32 for K <= 8192 with integer
    tokens, 119..133 is the range where the FP8 conversion is exact, and
    wider ranges reach the FP8 subnormals and the saturation;
  * tokens: "int" -> integers uniform on [-4, 4]; "normal" -> N(0, 1) cast to
    E4M3;
  * routing: `pairs` (token, expert) pairs drawn uniformly over the layer's
    experts (a multinomial count per expert); only experts with at least one
    row are listed, in a seeded random order, and their rows are contiguous
    in that order.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass
class MoeWorkload:
    name: str
    num_experts: int
    N: int
    K: int
    pairs: int            # routed (token, expert) pairs = rows of x
    scale_lo: int
    scale_hi: int
    x_kind: str           # "int" or "normal"
    seed: int


# A layer of the DSA model family's MoE: 256 routed experts, 8 per token,
# hidden size 7168, expert width 2048 with gate and up fused (N = 4096).
def decode_layer(seed: int = 11) -> MoeWorkload:
    """64 decode tokens x 8 experts = 512 rows over 256 experts."""
    return MoeWorkload("moe_decode_64tok_256e_n4096_k7168", 256, 4096, 7168, 512, 116, 124,
                       "normal", seed)


def prefill_layer(seed: int = 12) -> MoeWorkload:
    """An 8192-token prefill chunk x 8 experts = 65536 rows over 256 experts."""
    return MoeWorkload("moe_prefill_8192tok_256e_n4096_k7168", 256, 4096, 7168, 65536, 116,
                       124, "normal", seed)


def routing(wl: MoeWorkload):
    """(expert_ids int32 [n_act], row_offsets int32 [n_act + 1], max_rows)."""
    rng = np.random.default_rng([wl.seed, 1])
    counts = np.bincount(rng.integers(0, wl.num_experts, wl.pairs), minlength=wl.num_experts)
    order = rng.permutation(wl.num_experts)
    ids = np.array([e for e in order if counts[e] > 0], dtype=np.int32)
    rows = counts[ids]
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    return ids, offsets, int(rows.max())


def host_weights(wl: MoeWorkload, experts: Optional[np.ndarray] = None):
    """(codes uint8 [E, N, K/2], scales uint8 [E, N, K/32]) on the host; each
    expert's bytes depend only on (seed, expert), so a subset can be drawn."""
    ex = np.arange(wl.num_experts) if experts is None else np.asarray(experts)
    codes = np.empty((len(ex), wl.N, wl.K // 2), np.uint8)
    scales = np.empty((len(ex), wl.N, wl.K // 32), np.uint8)
    for j, e in enumerate(ex):
        rng = np.random.default_rng([wl.seed, 2, int(e)])
        codes[j] = rng.integers(0, 256, (wl.N, wl.K // 2), dtype=np.uint8)
        scales[j] = rng.integers(wl.scale_lo, wl.scale_hi + 1, (wl.N, wl.K // 32), dtype=np.uint8)
    return codes, scales


def host_tokens(wl: MoeWorkload, rows: Optional[int] = None):
    """E4M3 codes uint8 [pairs, K]."""
    import torch

    rng = np.random.default_rng([wl.seed, 3])
    M = wl.pairs if rows is None else rows
    if wl.x_kind == "int":
        v = torch.from_numpy(rng.integers(-4, 5, (M, wl.K)).astype(np.float32))
    else:
        v = torch.from_numpy(rng.standard_normal((M, wl.K)).astype(np.float32))
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def device_weights(wl: MoeWorkload, device="cuda"):
    """Full-size weights drawn on the device with torch's seeded generator
    (codes [E, N, K/2], scales [E, N, K/32]); host_weights draws different
    values -- full-size parity copies the sampled slices back instead."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000 + 2)
    codes = torch.randint(0, 256, (wl.num_experts, wl.N, wl.K // 2), dtype=torch.uint8,
                          device=device, generator=g)
    scales = torch.randint(wl.scale_lo, wl.scale_hi + 1, (wl.num_experts, wl.N, wl.K // 32),
                           dtype=torch.uint8, device=device, generator=g)
    return codes, scales


def device_tokens(wl: MoeWorkload, device="cuda"):
    """Full-size tokens drawn on the device: E4M3 codes uint8 [pairs, K]."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000 + 3)
    if wl.x_kind == "int":
        v = torch.randint(-4, 5, (wl.pairs, wl.K), device=device, generator=g).float()
    else:
        v = torch.randn((wl.pairs, wl.K), device=device, generator=g)
    return v.to(torch.float8_e4m3fn).view(torch.uint8)
