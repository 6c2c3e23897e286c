"""Seeded synthetic inputs for exact attention, shared by the tests, the bench and smoke().

This module holds no attention arithmetic: it draws Gaussian tensors, rounds them to the
storage dtype, and builds 128x128 block masks.  Both the fp64 oracle and the HIP path
receive exactly the arrays produced here.

Workload shapes follow the attention shapes of the workloads the pages name (BERT-large and
GPT-2 training, 16k/64k-token documents, block-sparse local+global patterns); the models and
datasets themselves are not used.  Page keys used in citations:

  [P1] "How FlashAttention Bypasses the GPU Memory Bottleneck to Enable Long-Context AI" (factlen.com)
  [P2] "FlashAttention: how a memory trick unlocked today's giant AI models" (khetwal.com)
  [P3] "How FlashAttention Eliminates Transformer Memory Bottlenecks" (Galileo blog)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MASK_BLOCK = 128  # block-mask granularity, the tile size of [P2 "A Worked Example in Pseudocode"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "fp32" or "bf16"
    causal: bool
    seed: int
    scale: float
    sparse: bool = False
    mask_seed: int | None = None
    fwd_only: bool = False
    description: str = ""

    @property
    def nb(self) -> int:
        return (self.N + MASK_BLOCK - 1) // MASK_BLOCK


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 1, 1, 256, 64, "fp32", False, 1001, 1.0 / math.sqrt(64),
                 description="tiny exact check, fp32, B=1 H=1 N=256 d=64"),
        Workload("bert", 8, 16, 512, 64, "bf16", False, 1002, 1.0 / 8.0,
                 description="BERT-large-shaped, B=8 H=16 N=512 d=64, non-causal"),
        Workload("gpt2", 8, 12, 2048, 64, "bf16", True, 1003, 1.0 / 8.0,
                 description="GPT-2-shaped causal, B=8 H=12 N=2048 d=64"),
        Workload("long", 1, 32, 16384, 128, "bf16", True, 1004, 1.0 / math.sqrt(128),
                 description="long-context causal, B=1 H=32 N=16384 d=128"),
        Workload("long64k", 1, 8, 65536, 128, "bf16", True, 1014, 1.0 / math.sqrt(128), fwd_only=True,
                 description="long-context causal forward, B=1 H=8 N=65536 d=128"),
        Workload("sparse", 4, 16, 8192, 64, "bf16", False, 1005, 1.0 / 8.0, sparse=True, mask_seed=2005,
                 description="block-sparse local(3)+global+10% random 128x128 mask, B=4 H=16 N=8192 d=64"),
    ]
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) with round-to-nearest-even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensors:
    """Inputs in storage form.  `q`, `k`, `v`, `do` are uint16 bf16 bit patterns for bf16 workloads
    and float32 for fp32 workloads, shape [B, H, N, d], row-major."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None
    dtype: str
    block_mask: np.ndarray | None = None
    extras: dict = field(default_factory=dict)

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def gaussian(shape, seed: int, count: int, dtype: str):
    """Draw `count` tensors of `shape` from N(0,1) with numpy's default_rng(seed), in order,
    as fp64 -> fp32 -> (bf16, round-to-nearest-even)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        x = rng.standard_normal(shape, dtype=np.float64).astype(np.float32)
        out.append(round_to_bf16_bits(x) if dtype == "bf16" else x)
    return out


def local_global_random_mask(nb: int, window: int, density: float, seed: int) -> np.ndarray:
    """uint8 [nb, nb] block mask: query block i attends key blocks i-window..i (local window),
    block 0 (global), and every other block independently with probability `density`."""
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    fixed = ((j <= i) & (j >= i - window)) | (j == 0)
    extra = np.random.default_rng(seed).random((nb, nb)) < density
    return (fixed | extra).astype(np.uint8)


def make(w: Workload | str, with_do: bool = True, B: int | None = None, H: int | None = None,
         N: int | None = None) -> Tensors:
    """Build the seeded inputs of a workload (optionally with a smaller B/H/N, same recipe)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    shape = (B, H, N, w.d)
    ts = gaussian(shape, w.seed, 4 if with_do else 3, w.dtype)
    mask = None
    if w.sparse:
        mask = local_global_random_mask((N + MASK_BLOCK - 1) // MASK_BLOCK, 3, 0.10, w.mask_seed)
    return Tensors(ts[0], ts[1], ts[2], ts[3] if with_do else None, w.dtype, mask)


def random_case(B: int, H: int, N: int, d: int, dtype: str, seed: int, with_do: bool = True,
                mask_density: float | None = None, mask_seed: int | None = None) -> Tensors:
    """Generic seeded case for sweeps (tiny N, ragged tails, edge cases)."""
    ts = gaussian((B, H, N, d), seed, 4 if with_do else 3, dtype)
    mask = None
    if mask_density is not None:
        nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
        rng = np.random.default_rng(mask_seed if mask_seed is not None else seed + 1)
        mask = (rng.random((nb, nb)) < mask_density).astype(np.uint8)
    return Tensors(ts[0], ts[1], ts[2], ts[3] if with_do else None, dtype, mask)


def flops_fwd(B: int, H: int, N: int, d: int, causal: bool, block_mask: np.ndarray | None = None) -> float:
    """Forward flop count convention: 4*B*H*N^2*d, halved for causal; block-sparse counts the
    active 128x128 blocks (4*B*H*d*128^2*nnz, intersected with causal if both)."""
    if block_mask is not None:
        nb = block_mask.shape[0]
        m = block_mask != 0
        if causal:
            m = m & np.tril(np.ones((nb, nb), dtype=bool))
        return 4.0 * B * H * d * MASK_BLOCK * MASK_BLOCK * float(m.sum())
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def flops_bwd(B, H, N, d, causal, block_mask=None) -> float:
    return 2.5 * flops_fwd(B, H, N, d, causal, block_mask)
