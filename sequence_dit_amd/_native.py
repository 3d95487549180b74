"""ctypes binding of ``libas_attn.so`` (include/as_attn.h).

Argument marshalling only: torch tensors become device pointers and sizes, the
current torch HIP stream becomes the ``stream`` argument, and outputs are
allocated with torch (caller-owned memory). Every step of the computation runs
in the library's HIP kernels; there is no CPU fallback, and a missing library
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libas_attn.so")

AS_OK, AS_ERR_INVALID_ARG, AS_ERR_UNSUPPORTED, AS_ERR_HIP = 0, 1, 2, 3
AS_BF16, AS_F32 = 0, 1
AS_MAX_PARTITIONS = 256
AS_MAX_MERGE = 64

EXPORTS = ("as_partition_attn", "as_merge", "as_partition_attn_states", "as_partition_attn_fp8",
           "as_merge_states", "as_compose_groups",
           "as_partition_contribution_workspace_size",
           "as_partition_contribution", "as_state_norms_workspace_size", "as_state_norms",
           "as_planner_decide", "as_planner_epsilon", "as_status_string", "as_last_error")

_lib = None


class ASError(RuntimeError):
    """A call into the library returned a status other than AS_OK."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


STATUS_NAMES = {AS_OK: "AS_OK", AS_ERR_INVALID_ARG: "AS_ERR_INVALID_ARG",
                AS_ERR_UNSUPPORTED: "AS_ERR_UNSUPPORTED", AS_ERR_HIP: "AS_ERR_HIP"}

c_i64p = ctypes.POINTER(ctypes.c_int64)
c_i32p = ctypes.POINTER(ctypes.c_int32)
c_vpp = ctypes.POINTER(ctypes.c_void_p)


def lib() -> ctypes.CDLL:
    """Load the library (once); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is missing: build it with "
                               "`python -m sequence_dit_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.as_partition_attn.restype = ctypes.c_int
        L.as_partition_attn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        c_i64p, c_i64p, c_i32p, ctypes.c_int32, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.as_merge.restype = ctypes.c_int
        L.as_merge.argtypes = [ctypes.c_int32, c_vpp, c_vpp, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.as_partition_attn_states.restype = ctypes.c_int
        L.as_partition_attn_states.argtypes = L.as_partition_attn.argtypes[:14] + [ctypes.c_int, ctypes.c_void_p,
                                                                                   ctypes.c_void_p, ctypes.c_void_p]
        L.as_partition_attn_fp8.restype = ctypes.c_int
        L.as_partition_attn_fp8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, c_i64p, c_i64p, c_i32p, ctypes.c_int32,
                                            ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]
        L.as_merge_states.restype = ctypes.c_int
        L.as_merge_states.argtypes = [ctypes.c_int32, c_vpp, c_vpp, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.as_compose_groups.restype = ctypes.c_int
        L.as_compose_groups.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
        L.as_partition_contribution_workspace_size.restype = ctypes.c_size_t
        L.as_partition_contribution_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64]
        L.as_partition_contribution.restype = ctypes.c_int
        L.as_partition_contribution.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                                ctypes.c_void_p]
        L.as_state_norms_workspace_size.restype = ctypes.c_size_t
        L.as_state_norms_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int64]
        L.as_state_norms.restype = ctypes.c_int
        L.as_state_norms.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.as_planner_decide.restype = ctypes.c_int
        L.as_planner_decide.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
        L.as_planner_epsilon.restype = ctypes.c_int
        L.as_planner_epsilon.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
        L.as_status_string.restype = ctypes.c_char_p
        L.as_status_string.argtypes = [ctypes.c_int]
        L.as_last_error.restype = ctypes.c_char_p
        L.as_last_error.argtypes = []
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != AS_OK:
        raise ASError(status, lib().as_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _require_gpu(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on a HIP device; the library has no CPU path")


def _i64(vals) -> ctypes.Array:
    return (ctypes.c_int64 * len(vals))(*vals)


# --------------------------------------------------------------------------- #
# as_partition_attn
# --------------------------------------------------------------------------- #

_STATE_DTYPES = {torch.float32: AS_F32, torch.bfloat16: AS_BF16}


def _state_code(dtype: torch.dtype) -> int:
    if dtype not in _STATE_DTYPES:
        raise ValueError("state OUT must be float32 or bfloat16")
    return _STATE_DTYPES[dtype]


def partition_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_ranges: Sequence[Tuple[int, int]],
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention states of q [B,H,Sq,D] against each range of k, v [B,H,Skv,D].

    Returns OUT [P,B,H,Sq,D] and LSE [P,B,H,Sq] (float32), enqueued on the current stream.
    """
    return _attn(q, k, v, kv_ranges, scale, out, lse, None)


def partition_attn_states(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_ranges: Sequence[Tuple[int, int]],
                          scale: Optional[float] = None, state_dtype: torch.dtype = torch.bfloat16,
                          out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """As partition_attn, with OUT stored as state_dtype (float32 or bfloat16); LSE is float32."""
    return _attn(q, k, v, kv_ranges, scale, out, lse, state_dtype)


def partition_attn_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_scale: torch.Tensor,
                       k_scale: torch.Tensor, kv_ranges: Sequence[Tuple[int, int]], scale: Optional[float] = None,
                       state_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention states from fp8 E4M3 queries and keys (torch.float8_e4m3fn, [B,H,Sq,D] and
    [B,H,Skv,D]) with float32 dequantisation factors q_scale, k_scale [B,H] (a code c of
    (b, h) stands for c * scale[b, h]) and bfloat16 values v (same shape and strides as k).
    Returns OUT [P,B,H,Sq,D] of state_dtype and LSE [P,B,H,Sq] float32."""
    _require_gpu(q, k, v, q_scale, k_scale)
    fp8 = torch.float8_e4m3fn
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("q must be [B,H,Sq,D]; k and v [B,H,Skv,D] with equal strides")
    if q.dtype != fp8 or k.dtype != fp8 or v.dtype != torch.bfloat16:
        raise ValueError("q and k must be float8_e4m3fn and v bfloat16")
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q and k/v disagree on B, H or D")
    if q.stride(3) != 1 or k.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    for t in (q_scale, k_scale):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != B * H:
            raise ValueError("q_scale and k_scale must be contiguous float32 [B, H]")
    Skv = k.shape[2]
    P = len(kv_ranges)
    code = _state_code(state_dtype)
    if out is None:
        out = torch.empty((P, B, H, Sq, D), dtype=state_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((P, B, H, Sq), dtype=torch.float32, device=q.device)
    if not (out.is_contiguous() and lse.is_contiguous() and out.dtype == state_dtype and lse.dtype == torch.float32):
        raise ValueError("out must be contiguous of the state dtype and lse contiguous float32")
    if out.numel() != P * B * H * Sq * D or lse.numel() != P * B * H * Sq:
        raise ValueError("out/lse have the wrong size")
    flat = [int(x) for r in kv_ranges for x in r]
    ranges = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    sc = float(D ** -0.5 if scale is None else scale)
    check(lib().as_partition_attn_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_scale.data_ptr(),
                                      k_scale.data_ptr(), B, H, Sq, Skv, D, _i64(q.stride()[:3]),
                                      _i64(k.stride()[:3]), ranges, P, sc, code, out.data_ptr(), lse.data_ptr(),
                                      _stream(q)))
    return out, lse


def _attn(q, k, v, kv_ranges, scale, out, lse, state_dtype):
    _require_gpu(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("q must be [B,H,Sq,D]; k and v [B,H,Skv,D] with equal strides")
    if q.dtype != k.dtype or k.dtype != v.dtype or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must share dtype bfloat16 or float32")
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q and k/v disagree on B, H or D")
    if q.stride(3) != 1 or k.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    Skv = k.shape[2]
    P = len(kv_ranges)
    odt = torch.float32 if state_dtype is None else state_dtype
    code = _state_code(odt)
    if out is None:
        out = torch.empty((P, B, H, Sq, D), dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty((P, B, H, Sq), dtype=torch.float32, device=q.device)
    if not (out.is_contiguous() and lse.is_contiguous() and out.dtype == odt and lse.dtype == torch.float32):
        raise ValueError("out must be contiguous of the state dtype and lse contiguous float32")
    if out.numel() != P * B * H * Sq * D or lse.numel() != P * B * H * Sq:
        raise ValueError("out/lse have the wrong size")
    flat = [int(x) for r in kv_ranges for x in r]
    ranges = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    dt = AS_BF16 if q.dtype == torch.bfloat16 else AS_F32
    sc = float(D ** -0.5 if scale is None else scale)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), dt, B, H, Sq, Skv, D,
            _i64(q.stride()[:3]), _i64(k.stride()[:3]), ranges, P, sc)
    if state_dtype is None:
        check(lib().as_partition_attn(*args, out.data_ptr(), lse.data_ptr(), _stream(q)))
    else:
        check(lib().as_partition_attn_states(*args, code, out.data_ptr(), lse.data_ptr(), _stream(q)))
    return out, lse


# --------------------------------------------------------------------------- #
# as_merge
# --------------------------------------------------------------------------- #

def merge(outs: Sequence[torch.Tensor], lses: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None,
          lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Compose n states (OUT_k [..., D], LSE_k [...]) into one; returns (OUT, LSE)."""
    n = len(outs)
    if n != len(lses) or n == 0:
        raise ValueError("need the same positive number of OUT and LSE tensors")
    _require_gpu(*outs, *lses)
    D = outs[0].shape[-1]
    rows = outs[0].numel() // D
    for o, l in zip(outs, lses):
        if o.dtype != torch.float32 or l.dtype != torch.float32 or not o.is_contiguous() or not l.is_contiguous():
            raise ValueError("states must be contiguous float32")
        if o.numel() != rows * D or l.numel() != rows:
            raise ValueError("states disagree in size")
    if out is None:
        out = torch.empty(outs[0].shape, dtype=torch.float32, device=outs[0].device)
    if lse is None:
        lse = torch.empty(lses[0].shape, dtype=torch.float32, device=outs[0].device)
    optrs = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    lptrs = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lses])
    check(lib().as_merge(n, optrs, lptrs, rows, D, out.data_ptr(), lse.data_ptr(), _stream(outs[0])))
    return out, lse


def merge_states(outs: Sequence[torch.Tensor], lses: Sequence[torch.Tensor], out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Compose n states whose OUT is float32 or bfloat16 (all the same); OUT written as out_dtype."""
    n = len(outs)
    if n != len(lses) or n == 0:
        raise ValueError("need the same positive number of OUT and LSE tensors")
    _require_gpu(*outs, *lses)
    in_dtype = outs[0].dtype
    in_code, out_code = _state_code(in_dtype), _state_code(out_dtype)
    D = outs[0].shape[-1]
    rows = outs[0].numel() // D
    for o, l in zip(outs, lses):
        if o.dtype != in_dtype or l.dtype != torch.float32 or not o.is_contiguous() or not l.is_contiguous():
            raise ValueError("states must be contiguous, OUT of one dtype, LSE float32")
        if o.numel() != rows * D or l.numel() != rows:
            raise ValueError("states disagree in size")
    if out is None:
        out = torch.empty(outs[0].shape, dtype=out_dtype, device=outs[0].device)
    if lse is None:
        lse = torch.empty(lses[0].shape, dtype=torch.float32, device=outs[0].device)
    optrs = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    lptrs = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lses])
    check(lib().as_merge_states(n, optrs, lptrs, in_code, rows, D, out_code, out.data_ptr(), lse.data_ptr(),
                                _stream(outs[0])))
    return out, lse


def compose_groups(outs: torch.Tensor, lses: torch.Tensor, group: int, out_dtype: Optional[torch.dtype] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Group-wise composition of a partition-major block of states OUT [P, ..., D], LSE [P, ...]:
    one state per group of `group` consecutive partitions ([G, ..., D], [G, ...])."""
    _require_gpu(outs, lses)
    if not outs.is_contiguous() or not lses.is_contiguous() or lses.dtype != torch.float32:
        raise ValueError("states must be contiguous with float32 LSE")
    in_code = _state_code(outs.dtype)
    out_dtype = outs.dtype if out_dtype is None else out_dtype
    out_code = _state_code(out_dtype)
    P, D = outs.shape[0], outs.shape[-1]
    rows = outs.numel() // max(P * D, 1)
    if lses.shape[0] != P or lses.numel() != P * rows:
        raise ValueError("OUT and LSE blocks disagree")
    G = (P + group - 1) // max(group, 1)
    if out is None:
        out = torch.empty((G,) + tuple(outs.shape[1:]), dtype=out_dtype, device=outs.device)
    if lse is None:
        lse = torch.empty((G,) + tuple(lses.shape[1:]), dtype=torch.float32, device=outs.device)
    check(lib().as_compose_groups(outs.data_ptr(), lses.data_ptr(), in_code, P, rows, D, group, out_code,
                                  out.data_ptr(), lse.data_ptr(), _stream(outs)))
    return out, lse


# --------------------------------------------------------------------------- #
# as_partition_contribution
# --------------------------------------------------------------------------- #

def contribution_workspace_size(P: int, rows: int, rows_per_group: int) -> int:
    return int(lib().as_partition_contribution_workspace_size(P, rows, rows_per_group))


def partition_contribution(lse: torch.Tensor, rows_per_group: int, want_weights: bool = True,
                           want_scores: bool = True, workspace: Optional[torch.Tensor] = None):
    """Per-row weights w [P, rows] and per-group scores [rows/rows_per_group, P] from LSE [P, ...]."""
    _require_gpu(lse)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32")
    P = lse.shape[0]
    rows = lse.numel() // max(P, 1)
    w = torch.empty((P, rows), dtype=torch.float32, device=lse.device) if want_weights else None
    s = None
    ws_bytes = 0
    if want_scores:
        if rows_per_group < 1 or rows % rows_per_group:
            raise ValueError("rows_per_group must divide the number of rows")
        s = torch.empty((rows // rows_per_group, P), dtype=torch.float32, device=lse.device)
        ws_bytes = contribution_workspace_size(P, rows, rows_per_group)
        if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=lse.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    check(lib().as_partition_contribution(lse.data_ptr(), P, rows, rows_per_group,
                                          w.data_ptr() if w is not None else None,
                                          s.data_ptr() if s is not None else None,
                                          workspace.data_ptr() if workspace is not None else None,
                                          ws_bytes, _stream(lse)))
    return w, s


# --------------------------------------------------------------------------- #
# Planner statistics: as_state_norms, as_planner_decide, as_planner_epsilon
# --------------------------------------------------------------------------- #

def state_norms_workspace_size(P: int, n: int) -> int:
    return int(lib().as_state_norms_workspace_size(P, n))


def _ptr(t: Optional[torch.Tensor]):
    return t.data_ptr() if t is not None else None


def state_norms(a: torch.Tensor, b: Optional[torch.Tensor] = None, norms: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """||a_i|| (or ||a_i - b_i||) for every slice i of a [P, ...] float32; returns norms [P] float32."""
    _require_gpu(a, *([b] if b is not None else []))
    if a.dtype != torch.float32 or not a.is_contiguous() or a.dim() < 1:
        raise ValueError("a must be a contiguous float32 tensor [P, ...]")
    if b is not None and (b.dtype != torch.float32 or not b.is_contiguous() or b.shape != a.shape):
        raise ValueError("b must be a contiguous float32 tensor shaped like a")
    P = a.shape[0]
    n = a.numel() // max(P, 1)
    if norms is None:
        norms = torch.empty(P, dtype=torch.float32, device=a.device)
    need = state_norms_workspace_size(P, n)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    check(lib().as_state_norms(a.data_ptr(), _ptr(b), P, n, norms.data_ptr(), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(a)))
    return norms


def planner_decide(anchor_norms: torch.Tensor, local_drift: torch.Tensor, weights: torch.Tensor,
                   eps: torch.Tensor, local: int, group: int, eps_local: float, want_stats: bool = True) -> dict:
    """One planning step (alpha, delta, group errors, compute flags, anchor flag), on the device."""
    _require_gpu(anchor_norms, local_drift, weights, eps)
    for t in (anchor_norms, local_drift, weights, eps):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("planner inputs must be contiguous float32")
    P = anchor_norms.numel()
    G = (P + group - 1) // max(group, 1)
    dev = anchor_norms.device
    r = {"compute": torch.empty(max(G, 1), dtype=torch.int32, device=dev),
         "anchor": torch.empty(1, dtype=torch.int32, device=dev)}
    if want_stats:
        r["alpha"] = torch.empty(P, dtype=torch.float32, device=dev)
        r["delta"] = torch.empty(P, dtype=torch.float32, device=dev)
        r["ase"] = torch.empty(max(G, 1), dtype=torch.float32, device=dev)
    check(lib().as_planner_decide(anchor_norms.data_ptr(), local_drift.data_ptr(), weights.data_ptr(),
                                  eps.data_ptr(), P, local, group, float(eps_local), _ptr(r.get("alpha")),
                                  _ptr(r.get("delta")), _ptr(r.get("ase")), r["compute"].data_ptr(),
                                  r["anchor"].data_ptr(), _stream(anchor_norms)))
    return r


def planner_epsilon(corr_norms: torch.Tensor, weights: torch.Tensor, local: int, group: int,
                    reuse_fraction: float, eps: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Reuse threshold of the anchor step from per-partition correction norms; returns eps [1]."""
    _require_gpu(corr_norms, weights)
    for t in (corr_norms, weights):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("planner inputs must be contiguous float32")
    if eps is None:
        eps = torch.empty(1, dtype=torch.float32, device=corr_norms.device)
    check(lib().as_planner_epsilon(corr_norms.data_ptr(), weights.data_ptr(), corr_norms.numel(), local, group,
                                   float(reuse_fraction), eps.data_ptr(), _stream(corr_norms)))
    return eps
