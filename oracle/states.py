"""fp64 reference definitions of attention states, their composition and partition weights.

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, the smoke check
and the bench's CPU-baseline leg are the only callers.

Sources (page titles as on the pages; no line numbers):

* DiTango review page (pith.science, arXiv 2607.15650), "What carries the
  argument": for KV partition i at denoising step t the attention state is
  AS_t(i) = (OUT_t(i), LSE_t(i)), the partial attention output and its
  log-sum-exp; states compose associatively and commutatively, so several
  remote partitions can be folded into one cached state.
* Same page, axiom ledger: the composition is the online-softmax identity of
  Eq. 1-2 (the equations themselves are not printed on the page).
* Same page, free-parameter ledger and Fig. 8 caption, Eq. 8: the partition
  importance w(i, t) is the softmax of the LSE values over partitions.
* Same page, "Core claim" and Fig. 6 caption: fresh states for high-contribution
  partitions, cached composed states for the others.
* Same page, "If this is right": a state is about half the size of the KV it
  summarises, and composed states can be merged into coarser groups under memory
  pressure (group-wise composition; group size g of 4, 8 or 16 in the
  free-parameter ledger).

Readings where the page is silent:

* scale tau = 1/sqrt(D) is an argument; LSE uses the natural log;
* OUT(i) is normalised within partition i (the only form in which (OUT, LSE)
  alone composes);
* an empty partition has the state (0, -inf), which is the identity of the
  composition; composing only empty states gives (0, -inf), never NaN;
* no attention mask (DiT joint self-attention);
* w(i) is taken per query row; the group score is the mean of w(i) over the
  rows of a group (one (batch, head) by default).

Everything is computed in float64 from the exact values handed to the GPU (bf16
inputs upcast, not the pre-rounding draws). Partition states use two passes
(max, then exponentials), not an online recurrence.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    """Upcast a numpy array or torch CPU tensor to float64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _workers() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _one_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """State of query rows q [Sq, D] against one partition's keys k, values v [n, D].

    z_j = scale * <q, k_j>; LSE = log sum_j exp(z_j); OUT = sum_j exp(z_j - LSE) v_j.
    """
    sq, d = q.shape
    if k.shape[0] == 0:
        return np.zeros((sq, v.shape[1])), np.full(sq, NEG_INF)
    z = scale * (q @ k.T)                       # [Sq, n]
    m = z.max(axis=1)                           # pass 1: row maximum
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    p = np.exp(z - lse[:, None])                # pass 2: normalised weights
    return p @ v, lse


def partition_states(q, k, v, kv_ranges: Sequence[Tuple[int, int]], scale: float,
                     workers: int | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention states of every query row against every KV range.

    q [B, H, Sq, D]; k, v [B, H, Skv, D]; kv_ranges = [(s_i, e_i)], 0 <= s_i <= e_i <= Skv.
    Returns OUT [P, B, H, Sq, D] and LSE [P, B, H, Sq] in float64.
    (DiTango review page, "What carries the argument": AS(i) = (OUT(i), LSE(i)).)
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Sq, D = q.shape
    P = len(kv_ranges)
    out = np.zeros((P, B, H, Sq, v.shape[-1]))
    lse = np.full((P, B, H, Sq), NEG_INF)

    def job(bh):
        b, h = bh
        for i, (s, e) in enumerate(kv_ranges):
            out[i, b, h], lse[i, b, h] = _one_state(q[b, h], k[b, h, s:e], v[b, h, s:e], scale)

    pairs = [(b, h) for b in range(B) for h in range(H)]
    n = workers or _workers()
    if n == 1 or len(pairs) == 1:
        for bh in pairs:
            job(bh)
    else:
        with ThreadPoolExecutor(max_workers=n) as pool:
            list(pool.map(job, pairs))
    return out, lse


def merge(outs, lses) -> Tuple[np.ndarray, np.ndarray]:
    """k-way composition of states (DiTango review page, axiom ledger, Eq. 1-2).

    outs [k, ..., D], lses [k, ...]. With M = max_k LSE_k:
      M = -inf           -> (0, -inf)   (every input empty)
      otherwise  a_k = exp(LSE_k - M), S = sum_k a_k,
                 LSE = M + log S,  OUT = sum_k (a_k / S) OUT_k.
    """
    outs, lses = _f64(outs), _f64(lses)
    M = lses.max(axis=0)
    empty = M == NEG_INF
    M0 = np.where(empty, 0.0, M)
    a = np.exp(lses - M0[None])                 # exp(-inf) = 0 for empty inputs
    S = a.sum(axis=0)
    S1 = np.where(empty, 1.0, S)
    lse = np.where(empty, NEG_INF, M0 + np.log(S1))
    weights = a / S1[None]
    out = (weights[..., None] * outs).sum(axis=0)
    out = np.where(empty[..., None], 0.0, out)
    return out, lse


def merge_pair(a: Tuple[np.ndarray, np.ndarray], b: Tuple[np.ndarray, np.ndarray]):
    """Composition of two states; the k = 2 case of ``merge``."""
    return merge(np.stack([_f64(a[0]), _f64(b[0])]), np.stack([_f64(a[1]), _f64(b[1])]))


def compose_groups(outs, lses, group: int) -> Tuple[np.ndarray, np.ndarray]:
    """Group-wise composition: the states of partitions k*group .. (k+1)*group - 1 (the
    last group may be shorter) merged into one state per group.

    outs [P, ..., D], lses [P, ...] -> [G, ..., D], [G, ...] with G = ceil(P / group).
    """
    outs, lses = _f64(outs), _f64(lses)
    P = outs.shape[0]
    parts = [merge(outs[k:k + group], lses[k:k + group]) for k in range(0, P, group)]
    return np.stack([o for o, _ in parts]), np.stack([l for _, l in parts])


def contribution(lse, rows_per_group: int) -> Tuple[np.ndarray, np.ndarray]:
    """Partition weights w and group scores from per-partition LSE.

    lse [P, rows]. Per row (DiTango review page, free-parameter ledger, Eq. 8:
    softmax of LSE over partitions): L* = log sum_i exp(LSE_i),
    w_i = exp(LSE_i - L*) (0 where LSE_i = -inf; all 0 if every LSE_i is -inf).
    scores[g][i] = mean of w_i over the rows_per_group rows of group g.
    Returns w [P, rows] and scores [rows / rows_per_group, P].
    """
    lse = _f64(lse)
    P, rows = lse.shape
    if rows % rows_per_group:
        raise ValueError("rows must be a multiple of rows_per_group")
    M = lse.max(axis=0)
    empty = M == NEG_INF
    M0 = np.where(empty, 0.0, M)
    S = np.exp(lse - M0[None]).sum(axis=0)
    lstar = np.where(empty, NEG_INF, M0 + np.log(np.where(empty, 1.0, S)))
    w = np.where(empty[None], 0.0, np.exp(lse - np.where(empty, 0.0, lstar)[None]))
    G = rows // rows_per_group
    scores = w.reshape(P, G, rows_per_group).mean(axis=2).T
    return w, scores


def full_attention(q, k, v, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of every query against all keys: OUT [B,H,Sq,D], LSE [B,H,Sq]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Skv = k.shape[2]
    out, lse = partition_states(q, k, v, [(0, Skv)], scale)
    return out[0], lse[0]


def nearest_partitions(P: int, local: int, count: int) -> List[int]:
    """Indices of the ``count`` partitions nearest to ``local`` by |i - local|, ties to the lower index.

    DiTango review page, "Core claim": nearby partitions dominate the output.
    """
    order = sorted(range(P), key=lambda i: (abs(i - local), i))
    return sorted(order[:count])


def selective_reuse(out_t, lse_t, out_t1, lse_t1, near: Sequence[int]):
    """One selective-reuse step (DiTango review page, "What carries the argument"; Fig. 6 caption).

    out_t/lse_t: states of all P partitions at step t (queries and keys of step t).
    out_t1/lse_t1: states at step t+1; only the ``near`` partitions are used.
    The partitions not in ``near`` are composed into one cached state C_t from
    step t; the result at t+1 composes the fresh near states with C_t.
    Returns (out, lse, cached_out, cached_lse).
    """
    out_t, lse_t = _f64(out_t), _f64(lse_t)
    P = out_t.shape[0]
    far = [i for i in range(P) if i not in set(near)]
    c_out, c_lse = merge(out_t[far], lse_t[far])
    fresh_out = _f64(out_t1)[list(near)]
    fresh_lse = _f64(lse_t1)[list(near)]
    r_out, r_lse = merge(np.concatenate([fresh_out, c_out[None]]), np.concatenate([fresh_lse, c_lse[None]]))
    return r_out, r_lse, c_out, c_lse


def mse(a, b) -> float:
    """Mean of squared differences over all elements."""
    return float(np.mean((_f64(a) - _f64(b)) ** 2))
