"""Selective attention-state reuse across denoising steps, as a sequence of library calls.

DiTango review page (pith.science), "What carries the argument" and Fig. 6 caption:
at an anchor step every partition's state is computed; the states of the
remote (low-contribution) partitions are composed into one cached state; at the
following steps only the near partitions are recomputed and composed with the
cached state. The partition weights (Eq. 8, softmax of LSE over partitions) are
refreshed at the anchor. The anchor-guided planner statistics (scale ratios,
drift model, group errors and the compute/reuse decision of Eqs. 9, 10, 12, 13)
are computed from the same buffers by ``plan_anchor`` and ``plan_step``.

Everything here is buffer management and ordering on the current torch stream;
each step of the arithmetic runs in the HIP library (``_native``).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import torch

from . import _native


def _v_scale(v: torch.Tensor, scales):
    """V's factors when v holds fp8 codes (scales = (q_scale, k_scale, v_scale)), else None."""
    if v.dtype != torch.float8_e4m3fn:
        return None
    if scales is None or len(scales) < 3:
        raise ValueError("fp8 v needs its dequantisation factors (scales = (q_scale, k_scale, v_scale))")
    return scales[2]


class SelectiveReuse:
    """Preallocated buffers and call order for one query shard against P partitions."""

    def __init__(self, B: int, H: int, Sq: int, D: int, ranges: Sequence[Tuple[int, int]], near: Sequence[int],
                 device, scale: float | None = None):
        # optional list that receives (name, start_event, end_event) around every library call
        # (or, with timer_only set, around the calls of those names only)
        self.timer: List | None = None
        self.timer_only: set | None = None
        self.ranges = [tuple(r) for r in ranges]
        self.P = len(self.ranges)
        self.near = sorted(int(i) for i in near)
        if not self.near or len(set(self.near)) != len(self.near) or not all(0 <= i < self.P for i in self.near):
            raise ValueError("near must be distinct partition indices")
        self.far = [i for i in range(self.P) if i not in set(self.near)]
        self.rows = B * H * Sq
        self.rows_per_group = Sq
        self.scale = D ** -0.5 if scale is None else scale
        f32 = dict(dtype=torch.float32, device=device)
        nf = len(self.near)
        # anchor: states of every partition
        self.state_out = torch.empty((self.P, B, H, Sq, D), **f32)
        self.state_lse = torch.empty((self.P, B, H, Sq), **f32)
        # reuse step: fresh near states plus the cached composed state in the last slot
        self.step_out = torch.empty((nf + 1, B, H, Sq, D), **f32)
        self.step_lse = torch.empty((nf + 1, B, H, Sq), **f32)
        self.result_out = torch.empty((B, H, Sq, D), **f32)
        self.result_lse = torch.empty((B, H, Sq), **f32)
        G = self.rows // self.rows_per_group
        self.anchor_weights = torch.empty((self.P, self.rows), **f32)
        self.anchor_scores = torch.empty((G, self.P), **f32)
        self.step_weights = torch.empty((nf + 1, self.rows), **f32)
        self.step_scores = torch.empty((G, nf + 1), **f32)
        ws = max(_native.contribution_workspace_size(self.P, self.rows, self.rows_per_group),
                 _native.contribution_workspace_size(nf + 1, self.rows, self.rows_per_group), 16)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        # planner: per-partition OUT norms and global weights at the anchor, local drift per step
        self.anchor_norms = torch.empty(self.P, **f32)
        self.global_weights = torch.empty((1, self.P), **f32)
        self.local_drift = torch.empty(1, **f32)
        n = self.rows * D
        self.norms_workspace = torch.empty(max(_native.state_norms_workspace_size(self.P, n),
                                               _native.state_norms_workspace_size(1, n), 16),
                                           dtype=torch.uint8, device=device)
        self.global_workspace = torch.empty(max(_native.contribution_workspace_size(self.P, self.rows, self.rows), 16),
                                            dtype=torch.uint8, device=device)

    @property
    def cached_out(self) -> torch.Tensor:
        return self.step_out[-1]

    @property
    def cached_lse(self) -> torch.Tensor:
        return self.step_lse[-1]

    def _timed(self, name: str, fn, *args, **kw):
        if self.timer is None or (self.timer_only is not None and name not in self.timer_only):
            return fn(*args, **kw)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        r = fn(*args, **kw)
        end.record()
        self.timer.append((name, start, end))
        return r

    def _attn(self, name: str, q, k, v, ranges, out, lse, scales) -> None:
        """Partition states: bf16 (or fp32) q/k/v, or fp8 E4M3 q/k with scales = (q_scale, k_scale),
        or fp8 q/k/v with scales = (q_scale, k_scale, v_scale)."""
        if q.dtype == torch.float8_e4m3fn:
            if scales is None:
                raise ValueError("fp8 q/k need their dequantisation factors (q_scale, k_scale)")
            if v.dtype == torch.float8_e4m3fn:
                self._timed(name, _native.partition_attn_fp8_qkv, q, k, v, scales[0], scales[1], scales[2], ranges,
                            self.scale, out=out, lse=lse)
            else:
                self._timed(name, _native.partition_attn_fp8, q, k, v, scales[0], scales[1], ranges, self.scale,
                            out=out, lse=lse)
        else:
            self._timed(name, _native.partition_attn, q, k, v, ranges, self.scale, out=out, lse=lse)

    def anchor(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scales=None) -> None:
        """Step t: all partition states, their weights, and the cached composition of the far ones.
        q and k (and v) may be fp8 E4M3 codes, with scales = (q_scale, k_scale[, v_scale]) float32 [B, H]."""
        self._attn("attn_anchor", q, k, v, self.ranges, self.state_out, self.state_lse, scales)
        self._timed("contrib_anchor", self._contribution, self.state_lse, self.anchor_weights, self.anchor_scores)
        self._timed("merge_cached", _native.merge, [self.state_out[i] for i in self.far],
                    [self.state_lse[i] for i in self.far], out=self.cached_out, lse=self.cached_lse)

    def step(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scales=None) -> Tuple[torch.Tensor, torch.Tensor]:
        """Step t+1: fresh near states composed with the cached state; returns (OUT, LSE).
        q and k may be fp8 E4M3 codes, with scales = (q_scale, k_scale) float32 [B, H]."""
        nf = len(self.near)
        self._attn("attn_fresh", q, k, v, [self.ranges[i] for i in self.near], self.step_out[:nf],
                   self.step_lse[:nf], scales)
        self._timed("merge_step", _native.merge, [self.step_out[j] for j in range(nf + 1)],
                    [self.step_lse[j] for j in range(nf + 1)], out=self.result_out, lse=self.result_lse)
        self._timed("contrib_step", self._contribution, self.step_lse, self.step_weights, self.step_scores)
        return self.result_out, self.result_lse

    # ------------------------------------------------------------------ #
    # Grouped launches: the partition-attention epilogue composes the states
    # ------------------------------------------------------------------ #

    def grouped_layout(self, far_group: int) -> Tuple[List[int], List[int]]:
        """Partition order and group starts of a grouped anchor: the far partitions in runs of
        `far_group` (composed in the kernel; long groups first), then every near partition alone."""
        order = list(self.far) + list(self.near)
        starts = list(range(0, len(self.far), far_group)) + [len(self.far) + i for i in range(len(self.near) + 1)]
        return order, starts

    def anchor_grouped(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, far_group: int = 4,
                       scales=None) -> None:
        """Step t with grouped launches: one launch gives the composed state of every run of
        `far_group` far partitions, the state of every near partition and the LSE of all partitions
        (weights from those); the cached state composes the far groups' states. The partition order
        of the weights and scores is grouped_layout's (far partitions first)."""
        order, starts = self.grouped_layout(far_group)
        G = len(starts) - 1
        n_far_groups = G - len(self.near)
        key = (far_group,)
        if getattr(self, "_grouped_key", None) != key:
            shape = self.state_out.shape[1:]
            self.group_out = torch.empty((G,) + tuple(shape), dtype=torch.float32, device=self.state_out.device)
            self.group_lse = torch.empty((G,) + tuple(self.state_lse.shape[1:]), dtype=torch.float32,
                                         device=self.state_out.device)
            self._grouped_key = key
        fp8 = scales is not None
        self._timed("attn_anchor_grouped", _native.partition_attn_grouped, q, k, v, [self.ranges[i] for i in order],
                    starts, self.scale, None, True, scales[0] if fp8 else None, scales[1] if fp8 else None,
                    self.group_out, self.group_lse, self.state_lse, v_scale=_v_scale(v, scales))
        self._timed("contrib_anchor", self._contribution, self.state_lse, self.anchor_weights, self.anchor_scores)
        self._timed("merge_cached_grouped", _native.merge, [self.group_out[g] for g in range(n_far_groups)],
                    [self.group_lse[g] for g in range(n_far_groups)], out=self.cached_out, lse=self.cached_lse)

    def step_grouped(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, near_group: int | None = None,
                     scales=None) -> Tuple[torch.Tensor, torch.Tensor]:
        """Step t+1 with grouped launches: the near partitions in runs of `near_group` (all of them
        by default), the cached state composed into the first group's result in the kernel; more
        than one group is then composed by as_merge. Every near partition's LSE goes to the weights."""
        nf = len(self.near)
        ng = nf if near_group is None else near_group
        starts = list(range(0, nf, ng)) + [nf]
        G = len(starts) - 1
        if getattr(self, "_step_group_key", None) != G:
            self.step_group_out = torch.empty((G,) + tuple(self.result_out.shape), dtype=torch.float32,
                                              device=self.result_out.device)
            self.step_group_lse = torch.empty((G,) + tuple(self.result_lse.shape), dtype=torch.float32,
                                              device=self.result_out.device)
            self._step_group_key = G
        fp8 = scales is not None
        dst_out, dst_lse = (self.result_out[None], self.result_lse[None]) if G == 1 else (self.step_group_out,
                                                                                          self.step_group_lse)
        self._timed("attn_fresh_grouped", _native.partition_attn_grouped, q, k, v,
                    [self.ranges[i] for i in self.near], starts, self.scale, (self.cached_out, self.cached_lse), True,
                    scales[0] if fp8 else None, scales[1] if fp8 else None, dst_out, dst_lse, self.step_lse[:nf],
                    v_scale=_v_scale(v, scales))
        if G > 1:
            self._timed("merge_step_grouped", _native.merge, list(self.step_group_out), list(self.step_group_lse),
                        out=self.result_out, lse=self.result_lse)
        self._timed("contrib_step", self._contribution, self.step_lse, self.step_weights, self.step_scores)
        return self.result_out, self.result_lse

    def plan_anchor(self) -> None:
        """Planner statistics of the anchor step: ||OUT(i)|| per partition and the global weights w(i)."""
        self._timed("plan_norms_anchor", _native.state_norms, self.state_out.view(self.P, -1),
                    norms=self.anchor_norms, workspace=self.norms_workspace)
        self._timed("plan_weights", self._global_weights)

    def plan_step(self, local: int, group: int, eps: torch.Tensor, eps_local: float) -> dict:
        """Planner decision at a reuse step: drift of the fresh local state from its anchor state, then
        alpha, delta, group errors and the per-group compute flags (the local partition must be near)."""
        fresh = self.step_out[self.near.index(local)]
        self._timed("plan_drift", _native.state_norms, fresh.view(1, -1), self.state_out[local].view(1, -1),
                    norms=self.local_drift, workspace=self.norms_workspace)
        return self._timed("plan_decide", _native.planner_decide, self.anchor_norms, self.local_drift,
                           self.global_weights.view(-1), eps, local, group, eps_local)

    def _global_weights(self) -> None:
        _native.check(_native.lib().as_partition_contribution(
            self.state_lse.data_ptr(), self.P, self.rows, self.rows, None, self.global_weights.data_ptr(),
            self.global_workspace.data_ptr(), self.global_workspace.numel(), _native._stream(self.state_lse)))

    def _contribution(self, lse: torch.Tensor, weights: torch.Tensor, scores: torch.Tensor) -> None:
        P = lse.shape[0]
        _native.check(_native.lib().as_partition_contribution(
            lse.data_ptr(), P, self.rows, self.rows_per_group, weights.data_ptr(), scores.data_ptr(),
            self.workspace.data_ptr(), self.workspace.numel(), _native._stream(lse)))

    def algorithmic_flops(self, D: int, Sq: int, B: int, H: int) -> Tuple[int, int]:
        """FLOP of the partition-attention launches (QK^T + PV) at the anchor and at a reuse step."""
        per_key = 4 * B * H * Sq * D
        full = sum(e - s for s, e in self.ranges) * per_key
        fresh = sum(self.ranges[i][1] - self.ranges[i][0] for i in self.near) * per_key
        return full, fresh
