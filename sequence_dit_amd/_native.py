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
AS_BF16, AS_F32, AS_FP8_E4M3 = 0, 1, 2
AS_MAX_PARTITIONS = 256
AS_MAX_MERGE = 64

EXPORTS = ("as_partition_attn", "as_merge", "as_partition_attn_states", "as_partition_attn_fp8",
           "as_partition_attn_fp8_qkv", "as_partition_attn_grouped", "as_state_bytes",
           "as_merge_states", "as_compose_groups",
           "as_partition_contribution_workspace_size",
           "as_partition_contribution", "as_partition_contribution_noalloc",
           "as_state_norms_workspace_size", "as_state_norms",
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
        _lib = load(LIB_PATH)
    return _lib


def load(path: str) -> ctypes.CDLL:
    """Open a build of the library at `path` with the C signatures declared."""
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is missing: build it with "
                           "`python -m sequence_dit_amd.build` (or __graft_entry__.build())")
    L = ctypes.CDLL(path)
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
    L.as_partition_attn_fp8_qkv.restype = ctypes.c_int
    L.as_partition_attn_fp8_qkv.argtypes = (L.as_partition_attn_fp8.argtypes[:5] + [ctypes.c_void_p]
                                            + L.as_partition_attn_fp8.argtypes[5:])
    L.as_state_bytes.restype = ctypes.c_size_t
    L.as_state_bytes.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
    L.as_partition_attn_grouped.restype = ctypes.c_int
    L.as_partition_attn_grouped.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, c_i64p, c_i64p, c_i32p,
                                            ctypes.c_int32, c_i32p, ctypes.c_int32, ctypes.c_float,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]
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
    L.as_partition_contribution_noalloc.restype = ctypes.c_int
    L.as_partition_contribution_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
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
    return L


def check(status: int) -> None:
    if status != AS_OK:
        raise ASError(status, lib().as_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _require_gpu(*ts: Optional[torch.Tensor]) -> None:
    """Every tensor whose pointer reaches the library lives on one HIP device (None is skipped)."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on a HIP device; the library has no CPU path")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors must live on one device (found {dev} and {t.device})")


def _check_buf(t: torch.Tensor, name: str, dtype: torch.dtype, numel: int) -> None:
    """A caller-supplied buffer the library reads or writes as `numel` contiguous elements of `dtype`."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, has {t.numel()}")


def _check_workspace(t: torch.Tensor, need: int) -> int:
    """A caller-supplied workspace of at least `need` bytes; returns its size in bytes."""
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = t.numel() * t.element_size()
    if nbytes < need:
        raise ValueError(f"workspace of {nbytes} bytes is smaller than the {need} bytes needed")
    return nbytes


def _ptr(t: Optional[torch.Tensor]):
    return t.data_ptr() if t is not None else None


def _i64(vals) -> ctypes.Array:
    return (ctypes.c_int64 * len(vals))(*vals)


# --------------------------------------------------------------------------- #
# as_partition_attn
# --------------------------------------------------------------------------- #

FP8 = torch.float8_e4m3fn
_STATE_DTYPES = {torch.float32: AS_F32, torch.bfloat16: AS_BF16, FP8: AS_FP8_E4M3}


def _state_code(dtype: torch.dtype) -> int:
    if dtype not in _STATE_DTYPES:
        raise ValueError("state OUT must be float32, bfloat16 or float8_e4m3fn (fp8 payloads)")
    return _STATE_DTYPES[dtype]


def state_bytes(state_dtype: torch.dtype, rows: int, D: int) -> int:
    """as_state_bytes: bytes of one state's OUT storage of rows x D."""
    n = int(lib().as_state_bytes(_state_code(state_dtype), rows, D))
    if n == 0 and rows * D > 0:
        raise ValueError(f"invalid state sizes rows={rows} D={D}")
    return n


class Fp8States:
    """A block of n fp8 state payloads (include/as_attn.h, "fp8 state payload"): ``data`` is
    uint8 [n, as_state_bytes(fp8, rows, D)]; state i's OUT[r, d] stands for
    decode(codes()[i, r, d]) * factors()[i, r]. ``shape`` is the logical shape of one state's
    OUT (rows = its product without D)."""

    dtype = FP8

    def __init__(self, data: torch.Tensor, shape: Sequence[int]):
        self.shape = tuple(int(x) for x in shape)
        self.D = self.shape[-1]
        self.rows = 1
        for x in self.shape[:-1]:
            self.rows *= x
        self.payload = state_bytes(FP8, self.rows, self.D)
        if data.dtype != torch.uint8 or data.dim() != 2 or data.shape[1] != self.payload or not data.is_contiguous():
            raise ValueError(f"fp8 state data must be contiguous uint8 [n, {self.payload}]")
        self.data = data

    @classmethod
    def empty(cls, n: int, shape: Sequence[int], device) -> "Fp8States":
        shape = tuple(int(x) for x in shape)
        rows = 1
        for x in shape[:-1]:
            rows *= x
        return cls(torch.empty((n, state_bytes(FP8, rows, shape[-1])), dtype=torch.uint8, device=device), shape)

    @property
    def n(self) -> int:
        return self.data.shape[0]

    @property
    def device(self):
        return self.data.device

    def __len__(self) -> int:
        return self.n

    def __getitem__(self, i: int) -> "Fp8States":
        if not -self.n <= i < self.n:
            raise IndexError(i)
        i %= self.n
        return Fp8States(self.data[i:i + 1], self.shape)

    def codes(self) -> torch.Tensor:
        """uint8 [n, *shape]: the E4M3 codes (a view)."""
        return self.data[:, :self.rows * self.D].view((self.n,) + self.shape)

    def factors(self) -> torch.Tensor:
        """float32 [n, *shape[:-1]]: the per-row factors (a view)."""
        off = self.rows * self.D
        return self.data[:, off:off + 4 * self.rows].view(torch.float32).view((self.n,) + self.shape[:-1])


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
                       state_dtype: torch.dtype = torch.float32, out=None,
                       lse: Optional[torch.Tensor] = None):
    """Attention states from fp8 E4M3 queries and keys (torch.float8_e4m3fn, [B,H,Sq,D] and
    [B,H,Skv,D]) with float32 dequantisation factors q_scale, k_scale [B,H] (a code c of
    (b, h) stands for c * scale[b, h]) and bfloat16 values v (same shape and strides as k).
    Returns OUT [P,B,H,Sq,D] of state_dtype (float8_e4m3fn: Fp8States of P payloads) and LSE
    [P,B,H,Sq] float32."""
    return _attn_fp8(q, k, v, q_scale, k_scale, None, kv_ranges, scale, state_dtype, out, lse)


def partition_attn_fp8_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_scale: torch.Tensor,
                           k_scale: torch.Tensor, v_scale: torch.Tensor, kv_ranges: Sequence[Tuple[int, int]],
                           scale: Optional[float] = None, state_dtype: torch.dtype = torch.float32, out=None,
                           lse: Optional[torch.Tensor] = None):
    """as_partition_attn_fp8_qkv: partition_attn_fp8 with fp8 E4M3 values too (v float8_e4m3fn,
    same shape and strides as k, factors v_scale [B,H])."""
    return _attn_fp8(q, k, v, q_scale, k_scale, v_scale, kv_ranges, scale, state_dtype, out, lse)


def _attn_fp8(q, k, v, q_scale, k_scale, v_scale, kv_ranges, scale, state_dtype, out, lse):
    v8 = v_scale is not None
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("q must be [B,H,Sq,D]; k and v [B,H,Skv,D] with equal strides")
    if q.dtype != FP8 or k.dtype != FP8 or v.dtype != (FP8 if v8 else torch.bfloat16):
        raise ValueError("q and k must be float8_e4m3fn and v " + ("float8_e4m3fn" if v8 else "bfloat16"))
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q and k/v disagree on B, H or D")
    if q.stride(3) != 1 or k.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    for t in (q_scale, k_scale) + ((v_scale,) if v8 else ()):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != B * H:
            raise ValueError("q_scale, k_scale and v_scale must be contiguous float32 [B, H]")
    Skv = k.shape[2]
    P = len(kv_ranges)
    code = _state_code(state_dtype)
    out, lse = _state_outputs(q, P, B, H, Sq, D, state_dtype, out, lse)
    _require_gpu(q, k, v, q_scale, k_scale, v_scale, _out_tensor(out), lse)
    flat = [int(x) for r in kv_ranges for x in r]
    ranges = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    sc = float(D ** -0.5 if scale is None else scale)
    head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr())
    tail = (B, H, Sq, Skv, D, _i64(q.stride()[:3]), _i64(k.stride()[:3]), ranges, P, sc, code,
            _out_tensor(out).data_ptr(), lse.data_ptr(), _stream(q))
    if v8:
        check(lib().as_partition_attn_fp8_qkv(*head, v_scale.data_ptr(), *tail))
    else:
        check(lib().as_partition_attn_fp8(*head, *tail))
    return out, lse


def _out_tensor(out):
    """The device tensor holding a state block's OUT (Fp8States: its payload bytes)."""
    return out.data if isinstance(out, Fp8States) else out


def _state_outputs(q, P, B, H, Sq, D, state_dtype, out, lse):
    """OUT [P,B,H,Sq,D] of state_dtype (fp8: Fp8States of P payloads) and LSE [P,B,H,Sq]
    float32: allocated, or the caller's checked."""
    if state_dtype == FP8:
        if out is None:
            out = Fp8States.empty(P, (B, H, Sq, D), q.device)
        if not isinstance(out, Fp8States) or out.n != P or out.rows != B * H * Sq or out.D != D:
            raise ValueError(f"out must be Fp8States of {P} states of {B * H * Sq} rows of {D}")
    else:
        if out is None:
            out = torch.empty((P, B, H, Sq, D), dtype=state_dtype, device=q.device)
        _check_buf(out, "out", state_dtype, P * B * H * Sq * D)
    if lse is None:
        lse = torch.empty((P, B, H, Sq), dtype=torch.float32, device=q.device)
    _check_buf(lse, "lse", torch.float32, P * B * H * Sq)
    return out, lse


def _attn(q, k, v, kv_ranges, scale, out, lse, state_dtype):
    fn, args, out, lse = _attn_call(q, k, v, kv_ranges, scale, out, lse, state_dtype)
    check(fn(*args))
    return out, lse


def prepare_partition_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_ranges: Sequence[Tuple[int, int]],
                           scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None):
    """partition_attn with its arguments checked and marshalled once: returns (launch, out, lse),
    where launch() enqueues the same as_partition_attn call on the stream current now. For
    repeated launches of one shape (timing short launches, whose per-call checks in Python
    would otherwise outlast them)."""
    fn, args, out, lse = _attn_call(q, k, v, kv_ranges, scale, out, lse, None)

    def launch() -> None:
        check(fn(*args))

    return launch, out, lse


def _attn_call(q, k, v, kv_ranges, scale, out, lse, state_dtype):
    """(C function, its arguments, out, lse) of a single-partition launch, checked."""
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
    out, lse = _state_outputs(q, P, B, H, Sq, D, odt, out, lse)
    _require_gpu(q, k, v, _out_tensor(out), lse)
    flat = [int(x) for r in kv_ranges for x in r]
    ranges = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    dt = AS_BF16 if q.dtype == torch.bfloat16 else AS_F32
    sc = float(D ** -0.5 if scale is None else scale)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), dt, B, H, Sq, Skv, D,
            _i64(q.stride()[:3]), _i64(k.stride()[:3]), ranges, P, sc)
    if state_dtype is None:
        return lib().as_partition_attn, args + (out.data_ptr(), lse.data_ptr(), _stream(q)), out, lse
    return (lib().as_partition_attn_states, args + (code, _out_tensor(out).data_ptr(), lse.data_ptr(), _stream(q)),
            out, lse)


def partition_attn_grouped(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_ranges: Sequence[Tuple[int, int]],
                           group_starts: Sequence[int], scale: Optional[float] = None,
                           fold: Optional[Tuple[torch.Tensor, torch.Tensor]] = None, want_part_lse: bool = True,
                           q_scale: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           part_lse: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None):
    """as_partition_attn_grouped: the composed state of every group of consecutive partitions
    (group g = partitions group_starts[g] .. group_starts[g+1]-1), OUT [G,B,H,Sq,D] and LSE [G,B,H,Sq]
    float32, and (want_part_lse) every partition's LSE [P,B,H,Sq]. q, k, v bfloat16, or q, k
    float8_e4m3fn codes with float32 factors q_scale, k_scale [B,H] and v bfloat16 (or v
    float8_e4m3fn codes too, with factors v_scale [B,H]). fold = (OUT
    [B,H,Sq,D], LSE [B,H,Sq]) float32 state composed into group 0's result. Returns (out, lse, part_lse)."""
    fp8 = q.dtype == torch.float8_e4m3fn
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("q must be [B,H,Sq,D]; k and v [B,H,Skv,D] with equal strides")
    v8 = fp8 and v.dtype == torch.float8_e4m3fn
    if fp8:
        if k.dtype != torch.float8_e4m3fn or v.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
            raise ValueError("fp8 q needs fp8 k and bfloat16 or fp8 v")
        if q_scale is None or k_scale is None or (v8 and v_scale is None):
            raise ValueError("fp8 q, k (and fp8 v) need their factors q_scale, k_scale (v_scale)")
    elif q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16 (or q, k float8_e4m3fn with bfloat16 v)")
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q and k/v disagree on B, H or D")
    if q.stride(3) != 1 or k.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    if fp8:
        for t in (q_scale, k_scale) + ((v_scale,) if v8 else ()):
            _check_buf(t, "q_scale/k_scale/v_scale", torch.float32, B * H)
    P, G = len(kv_ranges), len(group_starts) - 1
    if G < 1:
        raise ValueError("group_starts needs at least two entries")
    if out is None:
        out = torch.empty((G, B, H, Sq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((G, B, H, Sq), dtype=torch.float32, device=q.device)
    _check_buf(out, "out", torch.float32, G * B * H * Sq * D)
    _check_buf(lse, "lse", torch.float32, G * B * H * Sq)
    if want_part_lse:
        if part_lse is None:
            part_lse = torch.empty((P, B, H, Sq), dtype=torch.float32, device=q.device)
        _check_buf(part_lse, "part_lse", torch.float32, P * B * H * Sq)
    else:
        part_lse = None
    fo = fl = None
    if fold is not None:
        fo, fl = fold
        _check_buf(fo, "fold OUT", torch.float32, B * H * Sq * D)
        _check_buf(fl, "fold LSE", torch.float32, B * H * Sq)
    _require_gpu(q, k, v, q_scale if fp8 else None, k_scale if fp8 else None, v_scale if v8 else None, fo, fl, out,
                 lse, part_lse)
    flat = [int(x) for r in kv_ranges for x in r]
    ranges = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    starts = (ctypes.c_int32 * len(group_starts))(*[int(x) for x in group_starts])
    sc = float(D ** -0.5 if scale is None else scale)
    check(lib().as_partition_attn_grouped(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), AS_FP8_E4M3 if fp8 else AS_BF16,
        _ptr(q_scale) if fp8 else None, _ptr(k_scale) if fp8 else None, _ptr(v_scale) if v8 else None,
        B, H, Sq, k.shape[2], D,
        _i64(q.stride()[:3]), _i64(k.stride()[:3]), ranges, P, starts, G, sc, _ptr(fo), _ptr(fl),
        out.data_ptr(), lse.data_ptr(), _ptr(part_lse), _stream(q)))
    return out, lse, part_lse


# --------------------------------------------------------------------------- #
# as_merge
# --------------------------------------------------------------------------- #

def merge(outs: Sequence[torch.Tensor], lses: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None,
          lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Compose n states (OUT_k [..., D], LSE_k [...]) into one; returns (OUT, LSE)."""
    fn, args, out, lse = _merge_call(outs, lses, out, lse)
    check(fn(*args))
    return out, lse


def prepare_merge(outs: Sequence[torch.Tensor], lses: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None):
    """merge with its arguments checked and marshalled once: returns (launch, out, lse), where
    launch() enqueues the same as_merge call on the stream current now."""
    fn, args, out, lse = _merge_call(outs, lses, out, lse)

    def launch() -> None:
        check(fn(*args))

    return launch, out, lse


def _merge_call(outs, lses, out, lse):
    """(C function, its arguments, out, lse) of as_merge, checked."""
    n = len(outs)
    if n != len(lses) or n == 0:
        raise ValueError("need the same positive number of OUT and LSE tensors")
    D = outs[0].shape[-1]
    rows = outs[0].numel() // D
    for o, l in zip(outs, lses):
        _check_buf(o, "a state's OUT", torch.float32, rows * D)
        _check_buf(l, "a state's LSE", torch.float32, rows)
    if out is None:
        out = torch.empty(outs[0].shape, dtype=torch.float32, device=outs[0].device)
    if lse is None:
        lse = torch.empty(lses[0].shape, dtype=torch.float32, device=outs[0].device)
    _check_buf(out, "out", torch.float32, rows * D)
    _check_buf(lse, "lse", torch.float32, rows)
    _require_gpu(*outs, *lses, out, lse)
    optrs = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    lptrs = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lses])
    return lib().as_merge, (n, optrs, lptrs, rows, D, out.data_ptr(), lse.data_ptr(), _stream(outs[0])), out, lse


def _state_list(outs) -> Tuple[torch.dtype, int, int, Tuple[int, ...], List[int]]:
    """(dtype, rows, D, shape, device pointers) of a list of single states: tensors of one dtype
    and shape, or single-state Fp8States."""
    if isinstance(outs[0], Fp8States):
        shape = outs[0].shape
        for o in outs:
            if not isinstance(o, Fp8States) or o.n != 1 or o.shape != shape:
                raise ValueError("fp8 inputs must be single Fp8States of one shape")
        return FP8, outs[0].rows, outs[0].D, shape, [o.data.data_ptr() for o in outs]
    dt = outs[0].dtype
    _state_code(dt)
    D = outs[0].shape[-1]
    rows = outs[0].numel() // D
    for o in outs:
        _check_buf(o, "a state's OUT", dt, rows * D)
    return dt, rows, D, tuple(outs[0].shape), [o.data_ptr() for o in outs]


def merge_states(outs: Sequence, lses: Sequence[torch.Tensor], out_dtype: torch.dtype = torch.bfloat16,
                 out=None, lse: Optional[torch.Tensor] = None):
    """Compose n states whose OUT is float32, bfloat16 (tensors) or fp8 (single-state Fp8States),
    all of one kind; OUT written as out_dtype (float8_e4m3fn: a single-state Fp8States)."""
    n = len(outs)
    if n != len(lses) or n == 0:
        raise ValueError("need the same positive number of OUT and LSE tensors")
    in_dtype, rows, D, shape, ptrs = _state_list(outs)
    in_code, out_code = _state_code(in_dtype), _state_code(out_dtype)
    for l in lses:
        _check_buf(l, "a state's LSE", torch.float32, rows)
    dev = lses[0].device
    if out_dtype == FP8:
        if out is None:
            out = Fp8States.empty(1, shape, dev)
        if not isinstance(out, Fp8States) or out.n != 1 or out.rows != rows or out.D != D:
            raise ValueError("out must be a single Fp8States state of the inputs' shape")
    else:
        if out is None:
            out = torch.empty(shape, dtype=out_dtype, device=dev)
        _check_buf(out, "out", out_dtype, rows * D)
    if lse is None:
        lse = torch.empty(lses[0].shape, dtype=torch.float32, device=dev)
    _check_buf(lse, "lse", torch.float32, rows)
    _require_gpu(*[_out_tensor(o) for o in outs], *lses, _out_tensor(out), lse)
    optrs = (ctypes.c_void_p * n)(*ptrs)
    lptrs = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lses])
    check(lib().as_merge_states(n, optrs, lptrs, in_code, rows, D, out_code, _out_tensor(out).data_ptr(),
                                lse.data_ptr(), _stream(lses[0])))
    return out, lse


def compose_groups(outs, lses: torch.Tensor, group: int, out_dtype: Optional[torch.dtype] = None,
                   out=None, lse: Optional[torch.Tensor] = None):
    """Group-wise composition of a partition-major block of states OUT [P, ..., D] (or Fp8States
    of P states), LSE [P, ...]: one state per group of `group` consecutive partitions ([G, ..., D]
    or Fp8States of G states, [G, ...])."""
    fp8_in = isinstance(outs, Fp8States)
    in_dtype = FP8 if fp8_in else outs.dtype
    in_code = _state_code(in_dtype)
    out_dtype = in_dtype if out_dtype is None else out_dtype
    out_code = _state_code(out_dtype)
    if fp8_in:
        P, D, rows, shape = outs.n, outs.D, outs.rows, outs.shape
    else:
        P, D = outs.shape[0], outs.shape[-1]
        rows = outs.numel() // max(P * D, 1)
        shape = tuple(outs.shape[1:])
        _check_buf(outs, "outs", outs.dtype, P * rows * D)
    if lses.dim() < 1 or lses.shape[0] != P:
        raise ValueError("OUT and LSE blocks disagree")
    _check_buf(lses, "lses", torch.float32, P * rows)
    G = (P + group - 1) // max(group, 1)
    if out_dtype == FP8:
        if out is None:
            out = Fp8States.empty(G, shape, lses.device)
        if not isinstance(out, Fp8States) or out.n != G or out.rows != rows or out.D != D:
            raise ValueError(f"out must be Fp8States of {G} states of the inputs' shape")
    else:
        if out is None:
            out = torch.empty((G,) + shape, dtype=out_dtype, device=lses.device)
        _check_buf(out, "out", out_dtype, G * rows * D)
    if lse is None:
        lse = torch.empty((G,) + tuple(lses.shape[1:]), dtype=torch.float32, device=lses.device)
    _check_buf(lse, "lse", torch.float32, G * rows)
    _require_gpu(_out_tensor(outs), lses, _out_tensor(out), lse)
    check(lib().as_compose_groups(_out_tensor(outs).data_ptr(), lses.data_ptr(), in_code, P, rows, D, group, out_code,
                                  _out_tensor(out).data_ptr(), lse.data_ptr(), _stream(lses)))
    return out, lse


# --------------------------------------------------------------------------- #
# as_partition_contribution
# --------------------------------------------------------------------------- #

def contribution_workspace_size(P: int, rows: int, rows_per_group: int) -> int:
    return int(lib().as_partition_contribution_workspace_size(P, rows, rows_per_group))


def partition_contribution(lse: torch.Tensor, rows_per_group: int, want_weights: bool = True,
                           want_scores: bool = True, workspace: Optional[torch.Tensor] = None):
    """Per-row weights w [P, rows] and per-group scores [rows/rows_per_group, P] from LSE [P, ...]."""
    if lse.dim() < 1:
        raise ValueError("lse must be [P, ...]")
    P = lse.shape[0]
    rows = lse.numel() // max(P, 1)
    _check_buf(lse, "lse", torch.float32, P * rows)
    w = torch.empty((P, rows), dtype=torch.float32, device=lse.device) if want_weights else None
    s = None
    ws_bytes = 0
    if want_scores:
        if rows_per_group < 1 or rows % rows_per_group:
            raise ValueError("rows_per_group must divide the number of rows")
        s = torch.empty((rows // rows_per_group, P), dtype=torch.float32, device=lse.device)
        need = contribution_workspace_size(P, rows, rows_per_group)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=lse.device)
        ws_bytes = _check_workspace(workspace, need)
    else:
        workspace = None
    _require_gpu(lse, w, s, workspace)
    check(lib().as_partition_contribution(lse.data_ptr(), P, rows, rows_per_group,
                                          w.data_ptr() if w is not None else None,
                                          s.data_ptr() if s is not None else None,
                                          workspace.data_ptr() if workspace is not None else None,
                                          ws_bytes, _stream(lse)))
    return w, s


CONTRIBUTION_SCRATCH_BYTES = 1 << 20   # AS_CONTRIBUTION_SCRATCH_BYTES


def partition_contribution_noalloc(lse: torch.Tensor, rows_per_group: int, weights: Optional[torch.Tensor] = None,
                                   scores: Optional[torch.Tensor] = None):
    """as_partition_contribution_noalloc: weights [P, rows] and/or scores [rows/rows_per_group, P] written
    into caller tensors (either may be None), with no workspace and no allocation in the library."""
    if lse.dim() < 1:
        raise ValueError("lse must be [P, ...]")
    P = lse.shape[0]
    rows = lse.numel() // max(P, 1)
    _check_buf(lse, "lse", torch.float32, P * rows)
    if weights is not None:
        _check_buf(weights, "weights", torch.float32, P * rows)
    if scores is not None:
        if rows_per_group < 1 or rows % rows_per_group:
            raise ValueError("rows_per_group must divide the number of rows")
        _check_buf(scores, "scores", torch.float32, (rows // rows_per_group) * P)
    _require_gpu(lse, weights, scores)
    check(lib().as_partition_contribution_noalloc(lse.data_ptr(), P, rows, rows_per_group, _ptr(weights),
                                                  _ptr(scores), _stream(lse)))
    return weights, scores


# --------------------------------------------------------------------------- #
# Planner statistics: as_state_norms, as_planner_decide, as_planner_epsilon
# --------------------------------------------------------------------------- #

def state_norms_workspace_size(P: int, n: int) -> int:
    return int(lib().as_state_norms_workspace_size(P, n))


def state_norms(a: torch.Tensor, b: Optional[torch.Tensor] = None, norms: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """||a_i|| (or ||a_i - b_i||) for every slice i of a [P, ...] float32; returns norms [P] float32."""
    if a.dim() < 1:
        raise ValueError("a must be a tensor [P, ...]")
    P = a.shape[0]
    n = a.numel() // max(P, 1)
    _check_buf(a, "a", torch.float32, P * n)
    if b is not None:
        if b.shape != a.shape:
            raise ValueError("b must be shaped like a")
        _check_buf(b, "b", torch.float32, P * n)
    if norms is None:
        norms = torch.empty(P, dtype=torch.float32, device=a.device)
    _check_buf(norms, "norms", torch.float32, P)
    need = state_norms_workspace_size(P, n)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    ws_bytes = _check_workspace(workspace, need)
    _require_gpu(a, b, norms, workspace)
    check(lib().as_state_norms(a.data_ptr(), _ptr(b), P, n, norms.data_ptr(), workspace.data_ptr(),
                               ws_bytes, _stream(a)))
    return norms


def planner_decide(anchor_norms: torch.Tensor, local_drift: torch.Tensor, weights: torch.Tensor,
                   eps: torch.Tensor, local: int, group: int, eps_local: float, want_stats: bool = True) -> dict:
    """One planning step (alpha, delta, group errors, compute flags, anchor flag), on the device."""
    P = anchor_norms.numel()
    for t, name, numel in ((anchor_norms, "anchor_norms", P), (local_drift, "local_drift", 1),
                           (weights, "weights", P), (eps, "eps", 1)):
        _check_buf(t, name, torch.float32, numel)
    G = (P + min(group, P) - 1) // max(min(group, P), 1)
    dev = anchor_norms.device
    r = {"compute": torch.empty(max(G, 1), dtype=torch.int32, device=dev),
         "anchor": torch.empty(1, dtype=torch.int32, device=dev)}
    if want_stats:
        r["alpha"] = torch.empty(P, dtype=torch.float32, device=dev)
        r["delta"] = torch.empty(P, dtype=torch.float32, device=dev)
        r["ase"] = torch.empty(max(G, 1), dtype=torch.float32, device=dev)
    _require_gpu(anchor_norms, local_drift, weights, eps, *r.values())
    check(lib().as_planner_decide(anchor_norms.data_ptr(), local_drift.data_ptr(), weights.data_ptr(),
                                  eps.data_ptr(), P, local, group, float(eps_local), _ptr(r.get("alpha")),
                                  _ptr(r.get("delta")), _ptr(r.get("ase")), r["compute"].data_ptr(),
                                  r["anchor"].data_ptr(), _stream(anchor_norms)))
    return r


def planner_epsilon(corr_norms: torch.Tensor, weights: torch.Tensor, local: int, group: int,
                    reuse_fraction: float, eps: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Reuse threshold of the anchor step from per-partition correction norms; returns eps [1]."""
    P = corr_norms.numel()
    _check_buf(corr_norms, "corr_norms", torch.float32, P)
    _check_buf(weights, "weights", torch.float32, P)
    if eps is None:
        eps = torch.empty(1, dtype=torch.float32, device=corr_norms.device)
    _check_buf(eps, "eps", torch.float32, 1)
    _require_gpu(corr_norms, weights, eps)
    check(lib().as_planner_epsilon(corr_norms.data_ptr(), weights.data_ptr(), corr_norms.numel(), local, group,
                                   float(reuse_fraction), eps.data_ptr(), _stream(corr_norms)))
    return eps
