"""fp64 reference definitions of the anchor-guided planner statistics.

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, the smoke check
and the bench's CPU-baseline leg are the only callers.

Sources (page titles as on the pages; no line numbers):

* DiTango review page (pith.science), "What carries the argument": the planner
  decides per group of partitions whether to compute or reuse, from the error
  estimate ASE(G_i, t) = sum over the partitions j of the group of
  w(j, t) * delta(j, t, t_c) (Eq. 12), with w refreshed at anchor steps.
* Same page, free-parameter ledger: the partition scale ratio
  alpha(i) = ||AS_ta(i)|| / ||AS_ta(i_loc)|| measured at the anchor step (Eq. 9);
  the partition importance w(i, t) is the softmax of LSE over partitions (Eq. 8);
  the group size g (4, 8 or 16 explored); the local threshold eps_local triggers a
  new anchor when the local state drift exceeds it (Algorithm 1); the error
  threshold eps is a percentile of the anchor correction errors chosen to meet a
  target cache/compute ratio R (Algorithm 1).
* Same page, referee report (section 4.1.2): the drift model
  delta(i, t, t_a) = alpha(i) * ||AS_t(i_loc) - AS_ta(i_loc)||_2 (Eq. 10), and the
  reuse decision of Eq. 13 compares the estimate of Eq. 12 with the threshold.

Readings where the pages are silent:

* ||AS|| is the L2 (Frobenius) norm of the OUT part of the state over the whole
  query shard (every batch, head, query row and channel); LSE is not included;
* partitions form contiguous groups G_k = {k g, ..., k g + g - 1}; the last group
  may be shorter;
* a group is computed when ASE(G_k) > eps and reused otherwise; the group holding
  the local partition is always computed (its fresh state feeds the drift);
* a new anchor is due when the local drift exceeds eps_local;
* the anchor correction error of group k is E_k = sum over j in G_k of
  w(j) * ||OUT_ta(j) - OUT_tc(j)||, the error the cached states would have made at
  the anchor step; eps is the m-th smallest E_k over the non-local groups with
  m = floor(R * G') (G' non-local groups, R the target fraction of them to
  reuse), so that m of them fall at or below it; m = 0 gives eps = -inf (reuse
  nothing). m is computed as float32(R) * float32(G') rounded down, the same
  integer decision the GPU takes.
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def state_norm(a, b=None) -> np.ndarray:
    """||a_i|| (or ||a_i - b_i||) over everything but the leading partition axis, in fp64."""
    a = _f64(a)
    d = a if b is None else a - _f64(b)
    d = d.reshape(d.shape[0], -1)
    return np.sqrt(np.einsum("ij,ij->i", d, d))


def scale_ratios(anchor_norms: Sequence[float], local: int) -> np.ndarray:
    """alpha(i) = ||AS_ta(i)|| / ||AS_ta(i_loc)||  (Eq. 9)."""
    n = _f64(anchor_norms)
    return n / n[local]


def drift_errors(alpha, local_drift: float) -> np.ndarray:
    """delta(i, t, t_a) = alpha(i) * ||AS_t(i_loc) - AS_ta(i_loc)||  (Eq. 10)."""
    return _f64(alpha) * float(local_drift)


def groups(P: int, group: int):
    """Contiguous groups of `group` partitions; the last one may be shorter."""
    return [list(range(k, min(k + group, P))) for k in range(0, P, group)]


def group_errors(weights, delta, group: int) -> np.ndarray:
    """ASE(G_k, t) = sum over j in G_k of w(j) * delta(j)  (Eq. 12)."""
    w, d = _f64(weights), _f64(delta)
    return np.array([sum(w[j] * d[j] for j in g) for g in groups(len(w), group)])


def decide(ase, local: int, group: int, eps: float) -> np.ndarray:
    """Eq. 13: 1 = compute the group fresh, 0 = reuse its cached state; the local group is always computed."""
    ase = _f64(ase)
    compute = (ase > eps).astype(np.int32)
    compute[local // group] = 1
    return compute


def needs_anchor(local_drift: float, eps_local: float) -> bool:
    """Algorithm 1: a new anchor step when the local state drift exceeds eps_local."""
    return float(local_drift) > float(eps_local)


def reuse_count(reuse_fraction: float, n_groups: int) -> int:
    """m = floor(R * G'), computed in float32 and clamped to [0, G']."""
    m = math.floor(float(np.float32(reuse_fraction) * np.float32(n_groups)))
    return min(max(m, 0), n_groups)


def epsilon(corr_norms, weights, local: int, group: int, reuse_fraction: float) -> float:
    """Algorithm 1: eps = the m-th smallest anchor correction error of the non-local groups."""
    E = group_errors(weights, corr_norms, group)
    others = np.array([E[k] for k in range(len(E)) if k != local // group])
    m = reuse_count(reuse_fraction, len(others))
    if m == 0:
        return -math.inf
    return float(np.sort(others)[m - 1])


def planner(anchor_norms, local_drift: float, weights, local: int, group: int, eps: float,
            eps_local: float) -> dict:
    """All statistics of one planning step (Eqs. 9, 10, 12, 13 and the anchor trigger)."""
    alpha = scale_ratios(anchor_norms, local)
    delta = drift_errors(alpha, local_drift)
    ase = group_errors(weights, delta, group)
    return {"alpha": alpha, "delta": delta, "ase": ase, "compute": decide(ase, local, group, eps),
            "anchor": needs_anchor(local_drift, eps_local)}
