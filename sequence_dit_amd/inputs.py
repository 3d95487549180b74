"""Seeded synthetic inputs for the partition-attention workloads.

This module only draws random tensors and lays out key partitions. It holds
none of the attention-state arithmetic: the HIP path's callers and the CPU
oracle's tests both consume exactly the tensors produced here, so neither side
depends on the other.

Every draw comes from ``numpy.random.default_rng([workload_id, tensor_id])``
as float32 N(0, 1), is scaled, and (for bf16 workloads) is rounded once to
bfloat16 with round-to-nearest-even (torch's ``.to(torch.bfloat16)``). Both
sides receive the rounded tensor.

Tensor ids: 0 = Q, 1 = K, 2 = V, 3 = smooth-component parameters,
4/5/6 = next-step residuals of Q/K/V, 7 = merge-order permutation.

The five workloads follow the attention shapes of the DiT inference settings
on the pages (FastUSP page, abstract: FLUX-class image DiT; DiTango review page,
"Core claim" and Fig. 5/6 captions: video DiTs under context parallelism).
Real model activations are not available; the recipes below stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_SMOOTH = 0, 1, 2, 3
TENSOR_RQ, TENSOR_RK, TENSOR_RV, TENSOR_PERM = 4, 5, 6, 7

Range = Tuple[int, int]


@dataclass
class Workload:
    """One seeded attention workload: a local query shard against P KV ranges."""

    name: str
    B: int
    H: int
    Sq: int
    Skv: int
    D: int
    dtype: torch.dtype
    q: torch.Tensor  # [B, H, Sq, D], CPU
    k: torch.Tensor  # [B, H, Skv, D], CPU
    v: torch.Tensor  # [B, H, Skv, D], CPU
    ranges: List[Range]
    local: int  # index of the partition whose tokens form the query shard
    scale: float
    # next denoising step (selective-reuse workload only)
    q1: Optional[torch.Tensor] = None
    k1: Optional[torch.Tensor] = None
    v1: Optional[torch.Tensor] = None
    q8: Optional[torch.Tensor] = None        # fp8 E4M3 codes of q (fp8-input workloads)
    k8: Optional[torch.Tensor] = None
    q_scale: Optional[torch.Tensor] = None   # float32 [B, H]: a code stands for code * scale
    k_scale: Optional[torch.Tensor] = None
    near: List[int] = field(default_factory=list)
    merge_order: List[int] = field(default_factory=list)

    @property
    def P(self) -> int:
        return len(self.ranges)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.Sq


def rng(workload_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([workload_id, tensor_id])


def gaussian(workload_id: int, tensor_id: int, shape: Sequence[int], std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draw of ``shape`` from the (workload, tensor) stream."""
    x = rng(workload_id, tensor_id).standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def to_dtype(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype) if dtype != torch.float32 else t


def equal_ranges(total: int, parts: int) -> List[Range]:
    """Contiguous ranges of ceil(total/parts) keys; the last one takes the rest."""
    step = -(-total // parts)
    return [(min(i * step, total), min((i + 1) * step, total)) for i in range(parts)]


def random_ranges(seed: int, total: int, parts: int, max_len: int = 300) -> List[Range]:
    """`parts` seeded ranges inside [0, total): random starts and lengths below max_len, every
    17th one empty, every 23rd (from the 6th) a single key, the first one the whole sequence
    (so that ranges overlap)."""
    g = np.random.default_rng([seed, parts])
    s = g.integers(0, total, size=parts)
    n = g.integers(0, max_len, size=parts)
    n[::17] = 0
    n[5::23] = 1
    e = np.minimum(s + n, total)
    r = [(int(a), int(b)) for a, b in zip(s, e)]
    r[0] = (0, total)
    return r


def nearest_partitions(P: int, local: int, count: int) -> List[int]:
    """The ``count`` partitions closest to ``local`` by |i - local|, ties to the lower index."""
    order = sorted(range(P), key=lambda i: (abs(i - local), i))
    return sorted(order[:count])


# --------------------------------------------------------------------------- #
# Workload recipes
# --------------------------------------------------------------------------- #

def tiny_fp32() -> Workload:
    """B=1, H=1, D=64, 256 keys in 4 equal ranges, fp32 N(0,1); merged in a shuffled order."""
    wid = 1
    q = gaussian(wid, TENSOR_Q, (1, 1, 256, 64))
    k = gaussian(wid, TENSOR_K, (1, 1, 256, 64))
    v = gaussian(wid, TENSOR_V, (1, 1, 256, 64))
    order = rng(wid, TENSOR_PERM).permutation(4).tolist()
    return Workload("tiny fp32 oracle case (B1 H1 D64, 256 keys, P4)", 1, 1, 256, 256, 64, torch.float32,
                    to_dtype(q, torch.float32), to_dtype(k, torch.float32), to_dtype(v, torch.float32),
                    equal_ranges(256, 4), local=0, scale=64 ** -0.5, merge_order=order)


def image_dit() -> Workload:
    """FLUX-like: H=24, D=128, 512 text + 4096 image tokens, P=8, shard = partition 4 (576 tokens)."""
    wid, H, D, S, P = 2, 24, 128, 4608, 8
    ranges = equal_ranges(S, P)
    local = P // 2
    sq = ranges[local][1] - ranges[local][0]
    q = gaussian(wid, TENSOR_Q, (1, H, sq, D), 0.5)
    k = gaussian(wid, TENSOR_K, (1, H, S, D), 0.5)
    v = gaussian(wid, TENSOR_V, (1, H, S, D), 0.5)
    return Workload("image DiT (B1 H24 D128, 4608 keys, P8, shard 576)", 1, H, sq, S, D, torch.bfloat16,
                    to_dtype(q, torch.bfloat16), to_dtype(k, torch.bfloat16), to_dtype(v, torch.bfloat16),
                    ranges, local, D ** -0.5)


def video_dit() -> Workload:
    """CogVideoX-like: H=48, D=64, 226 text + 13x30x45 patches = 17776 tokens, P=8 of 2222, shard = partition 4."""
    wid, H, D, S, P = 3, 48, 64, 226 + 13 * 30 * 45, 8
    ranges = equal_ranges(S, P)
    local = P // 2
    sq = ranges[local][1] - ranges[local][0]
    q = gaussian(wid, TENSOR_Q, (1, H, sq, D))
    k = gaussian(wid, TENSOR_K, (1, H, S, D))
    v = gaussian(wid, TENSOR_V, (1, H, S, D))
    return Workload("video DiT (B1 H48 D64, 17776 keys, P8, shard 2222)", 1, H, sq, S, D, torch.bfloat16,
                    to_dtype(q, torch.bfloat16), to_dtype(k, torch.bfloat16), to_dtype(v, torch.bfloat16),
                    ranges, local, D ** -0.5)


LONG_FRAMES, LONG_HP, LONG_WP = 32, 48, 80
SMOOTH_RANK = 64


def smooth_basis(wid: int, H: int, D: int):
    """Parameters of a spatially smooth low-rank additive component for video tokens.

    Token t sits at frame f, row y, column x of a frames x 48 x 80 latent grid
    (t = f*48*80 + y*80 + x). phi(t) is a 64-dimensional random-Fourier feature
    of (f/3, y/24, x/40); per head, Q and K add a*phi(t)U_h and V adds a*phi(t)U'_h
    with U_h, U'_h having orthonormal rows and a = 3.5*D**0.25 (the scaled
    logit of a token with itself gains about a*a/sqrt(D) = 12.25). Nearby tokens get
    correlated queries and keys, so attention mass concentrates on nearby
    partitions, as the DiTango pages report for real video DiTs (DiTango review
    page, "Core claim"; Fig. 5 caption). The constants are this recipe's own.
    Returns (W [64,3], b [64], U [H,64,D], Uv [H,64,D], a).
    """
    g = rng(wid, TENSOR_SMOOTH)
    W = g.standard_normal((SMOOTH_RANK, 3))
    b = g.uniform(0.0, 2.0 * np.pi, SMOOTH_RANK)
    U = np.empty((H, SMOOTH_RANK, D))
    Uv = np.empty((H, SMOOTH_RANK, D))
    for h in range(H):
        U[h] = np.linalg.qr(g.standard_normal((D, SMOOTH_RANK)))[0].T
        Uv[h] = np.linalg.qr(g.standard_normal((D, SMOOTH_RANK)))[0].T
    return W, b, U, Uv, 3.5 * D ** 0.25


def smooth_features(W: np.ndarray, b: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """phi(t) for the given token indices, float32 [T, 64]."""
    f = tokens // (LONG_HP * LONG_WP)
    y = (tokens // LONG_WP) % LONG_HP
    x = tokens % LONG_WP
    coords = np.stack([f / 3.0, y / 24.0, x / 40.0], axis=1)
    return (np.sqrt(2.0 / SMOOTH_RANK) * np.cos(coords @ W.T + b)).astype(np.float32)


def long_video(frames: int = LONG_FRAMES, H: int = 24, P: int = 32, wid: int = 4) -> Workload:
    """Long video: H=24, D=128, 32 frames x 48 x 80 = 122880 tokens, P=32 (one frame each), shard = partition 16."""
    D = 128
    S = frames * LONG_HP * LONG_WP
    ranges = equal_ranges(S, P)
    local = P // 2
    s0, e0 = ranges[local]
    sq = e0 - s0
    W, b, U, Uv, a = smooth_basis(wid, H, D)
    phi = smooth_features(W, b, np.arange(S))
    aU = (a * U).astype(np.float32)
    aUv = (a * Uv).astype(np.float32)
    q = gaussian(wid, TENSOR_Q, (1, H, sq, D))
    k = gaussian(wid, TENSOR_K, (1, H, S, D))
    v = gaussian(wid, TENSOR_V, (1, H, S, D))
    for h in range(H):
        q[0, h] += phi[s0:e0] @ aU[h]
        k[0, h] += phi @ aU[h]
        v[0, h] += phi @ aUv[h]
    name = f"long video DiT (B1 H{H} D128, {S} keys, P{P}, shard {sq})"
    return Workload(name, 1, H, sq, S, D, torch.bfloat16,
                    to_dtype(q, torch.bfloat16), to_dtype(k, torch.bfloat16), to_dtype(v, torch.bfloat16),
                    ranges, local, D ** -0.5)


def next_step(w: Workload, wid: int, residual: float = 0.05) -> Workload:
    """Attach step t+1 inputs X' = round(float(X) + residual * N(0,1)) for X in Q, K, V."""
    def bump(t: torch.Tensor, tid: int) -> torch.Tensor:
        x = t.float().numpy() + gaussian(wid, tid, tuple(t.shape), residual)
        return to_dtype(x, w.dtype)
    w.q1 = bump(w.q, TENSOR_RQ)
    w.k1 = bump(w.k, TENSOR_RK)
    w.v1 = bump(w.v, TENSOR_RV)
    return w


def selective_reuse(frames: int = LONG_FRAMES, H: int = 24, P: int = 32, residual: float = 0.05,
                    fresh: int = 4) -> Workload:
    """Two denoising steps of the long-video workload; step t+1 recomputes the 4 nearest partitions."""
    w = long_video(frames, H, P)
    w = next_step(w, 5, residual)
    w.near = nearest_partitions(w.P, w.local, fresh)
    w.name = f"selective reuse, {w.name}, {fresh} fresh + {w.P - fresh} cached"
    return w


def small_case(seed: int, B: int, H: int, Sq: int, Skv: int, D: int, ranges: Sequence[Range],
               dtype: torch.dtype = torch.bfloat16, std: float = 1.0) -> Workload:
    """A small seeded case with arbitrary ranges (ragged, overlapping or empty), for parity tests."""
    wid = 1000 + seed
    q = gaussian(wid, TENSOR_Q, (B, H, Sq, D), std)
    k = gaussian(wid, TENSOR_K, (B, H, Skv, D), std)
    v = gaussian(wid, TENSOR_V, (B, H, Skv, D), std)
    return Workload(f"small case seed {seed}", B, H, Sq, Skv, D, dtype,
                    to_dtype(q, dtype), to_dtype(k, dtype), to_dtype(v, dtype),
                    list(ranges), 0, D ** -0.5)


FP8_MAX = 448.0   # largest finite E4M3 ("e4m3fn") magnitude


def quantize_fp8(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-(b, h) fp8 E4M3 codes of x [B, H, S, D] and float32 factors [B, H].

    factor = amax / 448 over the (b, h) slice (1 for an all-zero slice); codes are
    torch's float8_e4m3fn cast (round to nearest even) of x / factor, whose
    magnitude is at most 448 up to one fp32 rounding, so no code overflows. A code
    stands for its value times the factor of its (b, h).
    """
    xf = x.float()
    amax = xf.abs().amax(dim=(2, 3))
    factor = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).contiguous()
    codes = (xf / factor[:, :, None, None]).to(torch.float8_e4m3fn)
    return codes, factor


def small_case_fp8(seed: int, B: int, H: int, Sq: int, Skv: int, D: int, ranges: Sequence[Range],
                   std: float = 1.0) -> Workload:
    """small_case with fp8 codes attached: w.q8, w.k8, w.v8 (float8_e4m3fn) with their
    factors w.q_scale, w.k_scale, w.v_scale (float32 [B, H]); w.v stays the bf16 values
    (the fp8-q/k path takes those)."""
    w = small_case(seed, B, H, Sq, Skv, D, ranges, torch.bfloat16, std)
    w.q8, w.q_scale = quantize_fp8(w.q)
    w.k8, w.k_scale = quantize_fp8(w.k)
    w.v8, w.v_scale = quantize_fp8(w.v)
    w.name = f"fp8 {w.name}"
    return w


def with_fp8(w: Workload) -> Workload:
    """A workload with per-(b, h) fp8 codes of its q, k and v attached (as small_case_fp8)."""
    w.q8, w.q_scale = quantize_fp8(w.q)
    w.k8, w.k_scale = quantize_fp8(w.k)
    w.v8, w.v_scale = quantize_fp8(w.v)
    return w


TENSOR_FP8_STATE = 8


def random_fp8_states(seed: int, n: int, rows: int, D: int, n_empty: int = 0):
    """n fp8 state payload contents of rows x D, for composition tests: codes (uint8 [n, rows, D])
    drawn uniformly over the finite E4M3 codes (a NaN code is replaced by 0x7E), row factors
    (float32 [n, rows]) exp(N(0, 1)) / 256, LSE (float32 [n, rows]) 4 N(0, 1); n_empty random
    (state, row) pairs are empty states: codes 0, factor 0, LSE -inf."""
    g = np.random.default_rng([2000 + seed, TENSOR_FP8_STATE])
    codes = g.integers(0, 256, size=(n, rows, D), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    factors = (np.exp(g.standard_normal((n, rows))) / 256).astype(np.float32)
    lses = (g.standard_normal((n, rows)) * 4).astype(np.float32)
    if n_empty:
        idx = g.choice(n * rows, size=n_empty, replace=False)
        codes.reshape(n * rows, D)[idx] = 0
        factors.reshape(-1)[idx] = 0
        lses.reshape(-1)[idx] = -np.inf
    return codes, factors, lses


WORKLOADS = {1: tiny_fp32, 2: image_dit, 3: video_dit, 4: long_video, 5: selective_reuse}


def make(config: int) -> Workload:
    return WORKLOADS[config]()
