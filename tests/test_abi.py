"""C ABI checks that need no GPU: the library loads, exports every declared entry
point, and rejects invalid arguments on the host with the documented status and
a message, before any HIP call (no compute calls are made here)."""
import ctypes
import os
import re

import pytest

from sequence_dit_amd import _native as N

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "as_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(N.LIB_PATH), reason="libas_attn.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(as_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(N.EXPORTS), names
    L = N.lib()
    for name in names:
        assert hasattr(L, name), name


def test_diagnostics_build_is_separate():
    """The workgroup-stamp entry points exist only in the diagnostics library, which exports
    the same declared C ABI besides them."""
    from sequence_dit_amd import build, wg_stamps
    assert not hasattr(ctypes.CDLL(N.LIB_PATH), "as_debug_wg_stamps")
    if not os.path.exists(build.STAMPS_LIB_PATH):
        pytest.skip("diagnostics library not built")
    L = wg_stamps._load()
    for name in N.EXPORTS:
        getattr(L, name)


def test_status_strings():
    L = N.lib()
    assert L.as_status_string(N.AS_OK) == b"ok"
    assert b"invalid" in L.as_status_string(N.AS_ERR_INVALID_ARG)
    assert b"unsupported" in L.as_status_string(N.AS_ERR_UNSUPPORTED)
    assert b"HIP" in L.as_status_string(N.AS_ERR_HIP)


# Fake but aligned, non-null device addresses: validation never dereferences them,
# and every call below fails validation before reaching HIP.
FAKE = 0x10000


def attn(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, dtype=N.AS_BF16, B=1, H=2, Sq=16, Skv=64, D=128,
                qs=(4096, 2048, 128), kvs=(16384, 8192, 128), ranges=[(0, 32), (32, 64)],
                scale=0.088, out=FAKE, lse=FAKE)
    args.update(kw)
    rng = None
    if args["ranges"] is not None:
        flat = [x for r in args["ranges"] for x in r]
        rng = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    qs = N._i64(args["qs"]) if args["qs"] is not None else None
    kvs = N._i64(args["kvs"]) if args["kvs"] is not None else None
    P = args.get("P", len(args["ranges"]) if args["ranges"] is not None else 1)
    st = N.lib().as_partition_attn(args["q"], args["k"], args["v"], args["dtype"], args["B"], args["H"],
                                   args["Sq"], args["Skv"], args["D"], qs, kvs, rng, P, args["scale"],
                                   args["out"], args["lse"], None)
    return st, N.lib().as_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(q=0), N.AS_ERR_INVALID_ARG, "NULL"),
    (dict(out=0), N.AS_ERR_INVALID_ARG, "NULL"),
    (dict(dtype=7), N.AS_ERR_INVALID_ARG, "dtype"),
    (dict(B=-1), N.AS_ERR_INVALID_ARG, "negative"),
    (dict(D=0), N.AS_ERR_INVALID_ARG, "D="),
    (dict(D=96), N.AS_ERR_UNSUPPORTED, "bf16"),
    (dict(dtype=N.AS_F32, D=130, qs=(8320, 4160, 132), kvs=(8320, 4160, 132)), N.AS_ERR_UNSUPPORTED, "f32"),
    (dict(ranges=[(0, 65)]), N.AS_ERR_INVALID_ARG, "kv_ranges[0]"),
    (dict(ranges=[(10, 5)]), N.AS_ERR_INVALID_ARG, "kv_ranges[0]"),
    (dict(ranges=[(0, 4), (-1, 3)]), N.AS_ERR_INVALID_ARG, "kv_ranges[1]"),
    (dict(ranges=None, P=2), N.AS_ERR_INVALID_ARG, "kv_ranges is NULL"),
    (dict(ranges=[(0, 1)] * 257), N.AS_ERR_INVALID_ARG, "P=257"),
    (dict(scale=float("nan")), N.AS_ERR_INVALID_ARG, "scale"),
    (dict(scale=-1.0), N.AS_ERR_INVALID_ARG, "scale"),
    (dict(q=FAKE + 8), N.AS_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE + 4), N.AS_ERR_INVALID_ARG, "aligned"),
    (dict(qs=(4096, 2048, 100)), N.AS_ERR_INVALID_ARG, "multiples"),
    (dict(kvs=(16384, 8192, 64)), N.AS_ERR_INVALID_ARG, "smaller than D"),
    (dict(qs=None), N.AS_ERR_INVALID_ARG, "stride"),
    (dict(B=300, H=300), N.AS_ERR_UNSUPPORTED, "65535"),
])
def test_partition_attn_rejects(kw, status, text):
    st, msg = attn(**kw)
    assert st == status, msg
    assert text in msg


def test_partition_attn_empty_problem_is_ok_without_gpu():
    assert attn(Sq=0, q=0, out=0, lse=0)[0] == N.AS_OK
    assert attn(ranges=[], P=0)[0] == N.AS_OK


def merge_call(n=2, rows=8, D=128, outs=None, lses=None, out=FAKE, lse=FAKE + 0x200000):
    outs = outs if outs is not None else [FAKE + 0x1000 * (i + 1) for i in range(n)]
    lses = lses if lses is not None else [FAKE + 0x100000 + 0x1000 * i for i in range(n)]
    op = (ctypes.c_void_p * max(1, len(outs)))(*outs)
    lp = (ctypes.c_void_p * max(1, len(lses)))(*lses)
    st = N.lib().as_merge(n, op, lp, rows, D, out, lse, None)
    return st, N.lib().as_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(n=0), N.AS_ERR_INVALID_ARG, "n=0"),
    (dict(n=65), N.AS_ERR_INVALID_ARG, "n=65"),
    (dict(rows=-1), N.AS_ERR_INVALID_ARG, "negative"),
    (dict(D=6), N.AS_ERR_INVALID_ARG, "multiple of 4"),
    (dict(D=2048), N.AS_ERR_INVALID_ARG, "multiple of 4"),
    (dict(out=0), N.AS_ERR_INVALID_ARG, "NULL output"),
    (dict(out=FAKE + 8), N.AS_ERR_INVALID_ARG, "aligned"),
    (dict(outs=[FAKE + 0x1000, 0]), N.AS_ERR_INVALID_ARG, "input 1"),
    (dict(outs=[FAKE + 0x1000, FAKE + 0x2004]), N.AS_ERR_INVALID_ARG, "misaligned"),
    (dict(outs=[FAKE, FAKE + 0x2000]), N.AS_ERR_INVALID_ARG, "overlaps the output"),
    (dict(lse=FAKE), N.AS_ERR_INVALID_ARG, "out and lse overlap"),
])
def test_merge_rejects(kw, status, text):
    st, msg = merge_call(**kw)
    assert st == status, msg
    assert text in msg


def test_merge_zero_rows_ok_without_gpu():
    assert merge_call(rows=0)[0] == N.AS_OK


def test_contribution_workspace_size():
    L = N.lib()
    assert L.as_partition_contribution_workspace_size(32, 24 * 3840, 3840) == 24 * 15 * 32 * 4
    assert L.as_partition_contribution_workspace_size(4, 10, 5) == 2 * 1 * 4 * 4
    assert L.as_partition_contribution_workspace_size(4, 10, 3) == 0   # does not divide
    assert L.as_partition_contribution_workspace_size(0, 10, 5) == 0
    assert L.as_partition_contribution_workspace_size(257, 10, 5) == 0


def contrib_call(P=4, rows=64, rpg=16, lse=FAKE, w=FAKE, s=FAKE, ws=FAKE, wsb=1 << 20):
    st = N.lib().as_partition_contribution(lse, P, rows, rpg, w, s, ws, wsb, None)
    return st, N.lib().as_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(P=0), N.AS_ERR_INVALID_ARG, "P=0"),
    (dict(rows=-2), N.AS_ERR_INVALID_ARG, "negative"),
    (dict(rpg=0), N.AS_ERR_INVALID_ARG, "rows_per_group"),
    (dict(rpg=7), N.AS_ERR_INVALID_ARG, "multiple"),
    (dict(lse=0), N.AS_ERR_INVALID_ARG, "lse is NULL"),
    (dict(ws=0), N.AS_ERR_INVALID_ARG, "workspace is NULL"),
    (dict(wsb=4), N.AS_ERR_INVALID_ARG, "smaller"),
    (dict(ws=FAKE + 4), N.AS_ERR_INVALID_ARG, "aligned"),
])
def test_contribution_rejects(kw, status, text):
    st, msg = contrib_call(**kw)
    assert st == status, msg
    assert text in msg


def test_contribution_nothing_requested_ok_without_gpu():
    assert contrib_call(w=0, s=0, ws=0)[0] == N.AS_OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        N.partition_attn(x, x, x, [(0, 4)])


def test_state_norms_workspace_size():
    L = N.lib()
    # 32 partitions of a long-video shard (24 * 3840 rows x 128): chunks of 184320 floats -> 64 per slice
    n = 24 * 3840 * 128
    assert L.as_state_norms_workspace_size(32, n) == 32 * 64 * 8
    assert L.as_state_norms_workspace_size(1, 8) == 8            # one chunk
    assert L.as_state_norms_workspace_size(3, 0) == 3 * 8         # n = 0 still writes a zero partial
    assert L.as_state_norms_workspace_size(2, 6) == 0             # n not a multiple of 4
    assert L.as_state_norms_workspace_size(0, 8) == 0
    assert L.as_state_norms_workspace_size(257, 8) == 0


def norms_call(a=FAKE, b=0, P=2, n=1024, out=FAKE, ws=FAKE, wsb=1 << 20):
    st = N.lib().as_state_norms(a, b, P, n, out, ws, wsb, None)
    return st, N.lib().as_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(P=0), N.AS_ERR_INVALID_ARG, "P=0"),
    (dict(P=300), N.AS_ERR_INVALID_ARG, "P=300"),
    (dict(n=-4), N.AS_ERR_INVALID_ARG, "multiple of 4"),
    (dict(n=10), N.AS_ERR_INVALID_ARG, "multiple of 4"),
    (dict(out=0), N.AS_ERR_INVALID_ARG, "norms is NULL"),
    (dict(a=0), N.AS_ERR_INVALID_ARG, "a is NULL"),
    (dict(a=FAKE + 4), N.AS_ERR_INVALID_ARG, "16-byte"),
    (dict(b=FAKE + 8), N.AS_ERR_INVALID_ARG, "16-byte"),
    (dict(ws=0), N.AS_ERR_INVALID_ARG, "workspace is NULL"),
    (dict(wsb=8), N.AS_ERR_INVALID_ARG, "smaller"),
    (dict(ws=FAKE + 8), N.AS_ERR_INVALID_ARG, "aligned"),
])
def test_state_norms_rejects(kw, status, text):
    st, msg = norms_call(**kw)
    assert st == status, msg
    assert text in msg


def decide_call(an=FAKE, dr=FAKE, w=FAKE, eps=FAKE, P=8, local=3, group=2, eps_local=0.5,
                alpha=FAKE, delta=FAKE, ase=FAKE, comp=FAKE, anch=FAKE):
    st = N.lib().as_planner_decide(an, dr, w, eps, P, local, group, eps_local, alpha, delta, ase, comp, anch, None)
    return st, N.lib().as_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(P=0), N.AS_ERR_INVALID_ARG, "P=0"),
    (dict(local=8), N.AS_ERR_INVALID_ARG, "local=8"),
    (dict(local=-1), N.AS_ERR_INVALID_ARG, "local=-1"),
    (dict(group=0), N.AS_ERR_INVALID_ARG, "group=0"),
    (dict(eps_local=float("inf")), N.AS_ERR_INVALID_ARG, "eps_local"),
    (dict(eps_local=float("nan")), N.AS_ERR_INVALID_ARG, "eps_local"),
    (dict(an=0), N.AS_ERR_INVALID_ARG, "must not be NULL"),
    (dict(eps=0), N.AS_ERR_INVALID_ARG, "must not be NULL"),
    (dict(comp=0), N.AS_ERR_INVALID_ARG, "must not be NULL"),
    (dict(anch=0), N.AS_ERR_INVALID_ARG, "must not be NULL"),
    (dict(ase=FAKE + 2), N.AS_ERR_INVALID_ARG, "misaligned"),
])
def test_planner_decide_rejects(kw, status, text):
    st, msg = decide_call(**kw)
    assert st == status, msg
    assert text in msg


def epsilon_call(corr=FAKE, w=FAKE, P=8, local=3, group=2, R=0.5, eps=FAKE):
    st = N.lib().as_planner_epsilon(corr, w, P, local, group, R, eps, None)
    return st, N.lib().as_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(P=257), N.AS_ERR_INVALID_ARG, "P=257"),
    (dict(local=9), N.AS_ERR_INVALID_ARG, "local=9"),
    (dict(group=-1), N.AS_ERR_INVALID_ARG, "group=-1"),
    (dict(R=-0.1), N.AS_ERR_INVALID_ARG, "reuse_fraction"),
    (dict(R=1.5), N.AS_ERR_INVALID_ARG, "reuse_fraction"),
    (dict(R=float("nan")), N.AS_ERR_INVALID_ARG, "reuse_fraction"),
    (dict(corr=0), N.AS_ERR_INVALID_ARG, "must not be NULL"),
    (dict(eps=0), N.AS_ERR_INVALID_ARG, "must not be NULL"),
    (dict(w=FAKE + 1), N.AS_ERR_INVALID_ARG, "misaligned"),
])
def test_planner_epsilon_rejects(kw, status, text):
    st, msg = epsilon_call(**kw)
    assert st == status, msg
    assert text in msg


def test_planner_bindings_refuse_cpu_tensors():
    import torch
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="HIP device"):
        N.state_norms(x)
    with pytest.raises(ValueError, match="HIP device"):
        N.planner_epsilon(x[0], x[1], 0, 2, 0.5)


def test_partition_attn_states_rejects_bad_state_dtype():
    args = dict(q=FAKE, k=FAKE, v=FAKE, dtype=N.AS_BF16, B=1, H=2, Sq=16, Skv=64, D=128)
    flat = [0, 32, 32, 64]
    rng = (ctypes.c_int32 * 4)(*flat)
    st = N.lib().as_partition_attn_states(FAKE, FAKE, FAKE, N.AS_BF16, 1, 2, 16, 64, 128, N._i64((4096, 2048, 128)),
                                          N._i64((16384, 8192, 128)), rng, 2, 0.088, 7, FAKE, FAKE, None)
    assert st == N.AS_ERR_INVALID_ARG and "state_dtype" in N.lib().as_last_error().decode()


def merge_states_call(n=2, in_dt=N.AS_BF16, out_dt=N.AS_F32, rows=10, D=128, out=FAKE, lse=FAKE + 0x200000,
                      ptrs=None):
    ptrs = ptrs if ptrs is not None else [FAKE + 0x1000 * (i + 1) for i in range(max(n, 1))]
    optrs = (ctypes.c_void_p * len(ptrs))(*ptrs)
    lptrs = (ctypes.c_void_p * len(ptrs))(*ptrs)
    st = N.lib().as_merge_states(n, optrs, lptrs, in_dt, rows, D, out_dt, out, lse, None)
    return st, N.lib().as_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(in_dt=5), N.AS_ERR_INVALID_ARG, "state dtypes"),
    (dict(out_dt=-1), N.AS_ERR_INVALID_ARG, "state dtypes"),
    (dict(n=0), N.AS_ERR_INVALID_ARG, "n=0"),
    (dict(n=65, ptrs=[FAKE] * 65), N.AS_ERR_INVALID_ARG, "n=65"),
    (dict(D=6), N.AS_ERR_INVALID_ARG, "multiple of 4"),
    (dict(out=FAKE + 8), N.AS_ERR_INVALID_ARG, "16-byte"),
    (dict(ptrs=[FAKE + 4, FAKE + 0x2000]), N.AS_ERR_INVALID_ARG, "misaligned"),
    (dict(in_dt=N.AS_F32, ptrs=[FAKE + 8, FAKE + 0x2000]), N.AS_ERR_INVALID_ARG, "misaligned"),
    (dict(ptrs=[FAKE, FAKE + 0x1000], out=FAKE), N.AS_ERR_INVALID_ARG, "overlaps the output"),
])
def test_merge_states_rejects(kw, status, text):
    st, msg = merge_states_call(**kw)
    assert st == status, msg
    assert text in msg


def compose_call(outs=FAKE, lses=FAKE + 0x100000, in_dt=N.AS_F32, P=8, rows=16, D=128, group=4,
                 out_dt=N.AS_F32, out=FAKE + 0x200000, lse=FAKE + 0x300000):
    st = N.lib().as_compose_groups(outs, lses, in_dt, P, rows, D, group, out_dt, out, lse, None)
    return st, N.lib().as_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(in_dt=9), N.AS_ERR_INVALID_ARG, "state dtypes"),
    (dict(P=0), N.AS_ERR_INVALID_ARG, "P=0"),
    (dict(P=257), N.AS_ERR_INVALID_ARG, "P=257"),
    (dict(group=0), N.AS_ERR_INVALID_ARG, "group=0"),
    (dict(group=65), N.AS_ERR_INVALID_ARG, "group=65"),
    (dict(rows=-1), N.AS_ERR_INVALID_ARG, "negative"),
    (dict(D=2), N.AS_ERR_INVALID_ARG, "multiple of 4"),
    (dict(outs=0), N.AS_ERR_INVALID_ARG, "NULL"),
    (dict(out=FAKE + 0x200008), N.AS_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE + 0x1000), N.AS_ERR_INVALID_ARG, "overlap"),      # inside the 8 x 16 x 128 x 4 B input block
    (dict(lse=FAKE + 0x100010), N.AS_ERR_INVALID_ARG, "overlap"),   # inside the LSE block
])
def test_compose_groups_rejects(kw, status, text):
    st, msg = compose_call(**kw)
    assert st == status, msg
    assert text in msg


def test_compose_groups_zero_rows_ok_without_gpu():
    assert compose_call(rows=0)[0] == N.AS_OK


def attn_fp8(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, qsc=FAKE, ksc=FAKE, B=1, H=2, Sq=16, Skv=64, D=128,
                qs=(4096, 2048, 128), kvs=(16384, 8192, 128), ranges=[(0, 32), (32, 64)],
                scale=0.088, state=N.AS_F32, out=FAKE, lse=FAKE)
    args.update(kw)
    flat = [x for r in args["ranges"] for x in r]
    rng = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    st = N.lib().as_partition_attn_fp8(args["q"], args["k"], args["v"], args["qsc"], args["ksc"], args["B"],
                                       args["H"], args["Sq"], args["Skv"], args["D"], N._i64(args["qs"]),
                                       N._i64(args["kvs"]), rng, len(args["ranges"]), args["scale"],
                                       args["state"], args["out"], args["lse"], None)
    return st, N.lib().as_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(qsc=0), N.AS_ERR_INVALID_ARG, "q_scale and k_scale"),
    (dict(ksc=0), N.AS_ERR_INVALID_ARG, "q_scale and k_scale"),
    (dict(ksc=FAKE + 2), N.AS_ERR_INVALID_ARG, "4-byte aligned"),
    (dict(D=96, qs=(3072, 1536, 96), kvs=(12288, 6144, 96)), N.AS_ERR_UNSUPPORTED, "fp8"),
    (dict(qs=(4096, 2048, 136)), N.AS_ERR_INVALID_ARG, "multiples of 16"),
    (dict(kvs=(16384, 8192, 136)), N.AS_ERR_INVALID_ARG, "multiples of 16"),
    (dict(state=7), N.AS_ERR_INVALID_ARG, "state_dtype"),
    (dict(q=FAKE + 8), N.AS_ERR_INVALID_ARG, "aligned"),
    (dict(ranges=[(0, 65)]), N.AS_ERR_INVALID_ARG, "kv_ranges[0]"),
])
def test_partition_attn_fp8_rejects(kw, status, text):
    st, msg = attn_fp8(**kw)
    assert st == status, msg
    assert text in msg


def test_partition_attn_fp8_empty_problem_is_ok_without_gpu():
    assert attn_fp8(Sq=0, q=0, out=0, lse=0, qsc=0, ksc=0)[0] == N.AS_OK


# --------------------------------------------------------------------------- #
# Aliasing: every output is checked against every input (and the other outputs)
# on byte ranges, partial overlaps included; overlapping calls fail before any HIP call.
# --------------------------------------------------------------------------- #

QA, KA, VA, OA, LA = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
# extents with the attn() shapes (B1 H2 Sq16 Skv64 D128, bf16): q 8192 B, k and v 32768 B,
# out 2 x 32 x 128 x 4 = 32768 B, lse 256 B


@pytest.mark.parametrize("kw,text", [
    (dict(out=QA + 0x1000), "overlaps input q"),            # starts inside q
    (dict(out=QA - 0x4000), "overlaps input q"),            # covers q's start
    (dict(lse=VA + 0x7ff0), "overlaps input v"),            # last 16 bytes of v
    (dict(lse=KA), "overlaps input k"),
    (dict(lse=OA + 0x7f00), "out and lse overlap"),
    (dict(out=QA + 16000, qs=(8192, 4096, 256)), "overlaps input q"),   # inside a strided q's span
])
def test_partition_attn_rejects_overlapping_outputs(kw, text):
    args = dict(q=QA, k=KA, v=VA, out=OA, lse=LA)
    args.update(kw)
    st, msg = attn(**args)
    assert st == N.AS_ERR_INVALID_ARG, msg
    assert text in msg


def test_partition_attn_fp8_rejects_overlapping_outputs():
    # fp8 q is 1 byte per element: B1 H2 Sq16 D128 with strides (4096, 2048, 128) spans 4096 bytes
    st, msg = attn_fp8(q=QA, k=KA, v=VA, qsc=0x600000, ksc=0x700000, out=QA + 4080, lse=LA)
    assert st == N.AS_ERR_INVALID_ARG and "overlaps input q" in msg, msg
    st, msg = attn_fp8(q=QA, k=KA, v=VA, qsc=0x600000, ksc=0x700000, out=OA, lse=OA + 0x10)
    assert st == N.AS_ERR_INVALID_ARG and "out and lse overlap" in msg, msg


def test_partition_attn_rejects_short_range_with_huge_stride():
    """A tile reads up to 128 key rows from a range's start (past a shorter range's end, where the
    hardware range check returns zeros): their 32-bit byte offsets must not wrap."""
    st, msg = attn(q=QA, k=KA, v=VA, out=OA, lse=LA, Skv=2, ranges=[(0, 1)], kvs=(1 << 25, 1 << 24, 1 << 24))
    assert st == N.AS_ERR_UNSUPPORTED and "2^31" in msg, msg


def test_partition_attn_rejects_sizes_whose_products_overflow():
    st, msg = attn(B=1 << 40, H=1 << 40)
    assert st == N.AS_ERR_UNSUPPORTED and "65535" in msg, msg


@pytest.mark.parametrize("kw,text", [
    (dict(out=FAKE + 0x1000 + 64 * 4), "input 0 overlaps the output"),      # 64 floats into input 0's OUT
    (dict(out=FAKE + 0x100000 - 0x800), "input 0 overlaps the output"),     # out's tail covers input 0's LSE
    (dict(lse=FAKE + 0x2000 + 0xff0), "input 1 overlaps the output"),       # lse inside input 1's OUT
    (dict(lse=FAKE + 0x101000 + 4), "input 1 overlaps the output"),         # lse one float into input 1's LSE
])
def test_merge_rejects_partial_overlaps(kw, text):
    # inputs: OUT at FAKE + 0x1000 (i + 1) (8 rows x 128 x 4 = 4 KiB each), LSE at FAKE + 0x100000 + 0x1000 i
    st, msg = merge_call(**kw)
    assert st == N.AS_ERR_INVALID_ARG, msg
    assert text in msg


def test_merge_states_rejects_partial_overlap():
    # bf16 inputs of 10 rows x 128 x 2 = 2560 bytes at FAKE + 0x1000 (i + 1); LSE blocks alias the OUT pointers
    st, msg = merge_states_call(out=FAKE + 0x2000 + 0x900)
    assert st == N.AS_ERR_INVALID_ARG and "overlaps the output" in msg, msg


@pytest.mark.parametrize("kw", [dict(w=FAKE + 0x100), dict(s=FAKE + 0x40), dict(ws=FAKE),
                                dict(lse=0x200000, w=0x300000, s=0x400000, ws=0x400010)])
def test_contribution_rejects_overlaps(kw):
    args = dict(lse=FAKE, w=0x200000, s=0x300000, ws=0x400000)
    args.update(kw)
    st, msg = contrib_call(**args)
    assert st == N.AS_ERR_INVALID_ARG and "must not overlap" in msg, msg


@pytest.mark.parametrize("kw", [dict(out=FAKE + 0x100), dict(b=0x300000, out=0x300000 + 0x1000),
                                dict(ws=FAKE + 0x1000), dict(ws=0x200000 - 0x10, out=0x200000 - 4)])
def test_state_norms_rejects_overlaps(kw):
    args = dict(a=FAKE, out=0x200000, ws=0x400000)
    args.update(kw)
    st, msg = norms_call(**args)
    assert st == N.AS_ERR_INVALID_ARG and "overlap" in msg, msg


def test_planner_rejects_overlaps():
    base = dict(an=0x100000, dr=0x110000, w=0x120000, eps=0x130000, alpha=0x140000, delta=0x150000,
                ase=0x160000, comp=0x170000, anch=0x180000)
    for kw in (dict(alpha=0x100000 + 16), dict(comp=0x120000), dict(anch=0x160000 + 4), dict(delta=0x140000 + 8)):
        args = dict(base)
        args.update(kw)
        st, msg = decide_call(**args)
        assert st == N.AS_ERR_INVALID_ARG and "overlap" in msg, (kw, msg)
    st, msg = epsilon_call(corr=0x100000, w=0x120000, eps=0x100000 + 8)
    assert st == N.AS_ERR_INVALID_ARG and "overlaps" in msg, msg


# --------------------------------------------------------------------------- #
# The Python binding: every tensor whose pointer reaches the library goes through the
# device check, and caller-supplied outputs of the wrong dtype, layout or size are
# refused before any library call. The library is replaced by a recorder here.
# --------------------------------------------------------------------------- #

class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        if name.endswith("_workspace_size"):
            return lambda *a: 64
        if name == "as_last_error":
            return lambda: b""

        def call(*args):
            self.calls.append((name, args))
            return N.AS_OK
        return call


def _pointers(args):
    ptrs = []
    for a in args:
        if isinstance(a, ctypes.Array) and a._type_ is ctypes.c_void_p:
            ptrs.extend(int(x) for x in a if x)
        elif isinstance(a, int) and a > 4096:
            ptrs.append(a)
    return ptrs


@pytest.fixture
def recorded(monkeypatch):
    import torch
    rec = _Recorder()
    checked = set()

    def require_gpu(*ts):
        for t in ts:
            if t is not None:
                checked.add(t.data_ptr())

    monkeypatch.setattr(N, "_lib", rec)
    monkeypatch.setattr(N, "_require_gpu", require_gpu)
    monkeypatch.setattr(N, "_stream", lambda t: 0)
    return torch, rec, checked


def test_binding_device_checks_cover_every_pointer(recorded):
    torch, rec, checked = recorded
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros(1, 2, 8, 64, dtype=bf)
    kv = torch.zeros(1, 2, 32, 64, dtype=bf)
    out = torch.zeros(2, 1, 2, 8, 64)
    lse = torch.zeros(2, 1, 2, 8)
    N.partition_attn(q, kv, kv.clone(), [(0, 16), (16, 32)], out=out, lse=lse)
    N.partition_attn_states(q, kv, kv.clone(), [(0, 16), (16, 32)], state_dtype=bf)
    q8, k8 = q.to(torch.float8_e4m3fn), kv.to(torch.float8_e4m3fn)
    N.partition_attn_fp8(q8, k8, kv, torch.ones(1, 2), torch.ones(1, 2), [(0, 32)])
    states, lses = torch.zeros(3, 16, 64), torch.zeros(3, 16)
    N.merge(list(states), list(lses))
    N.merge_states(list(states.to(bf)), list(lses), f32)
    N.compose_groups(states, lses, 2)
    N.partition_contribution(lses, 8)
    N.state_norms(states.view(3, -1), torch.ones(3, 16 * 64))
    N.planner_decide(torch.ones(4), torch.ones(1), torch.ones(4), torch.ones(1), 1, 2, 0.5)
    N.planner_epsilon(torch.ones(4), torch.ones(4), 1, 2, 0.5)
    assert len(rec.calls) == 10, [c[0] for c in rec.calls]
    for name, args in rec.calls:
        missing = [p for p in _pointers(args) if p not in checked]
        assert not missing, f"{name}: pointers {missing} skipped the device check"


@pytest.mark.parametrize("case", ["attn_out_small", "attn_out_dtype", "attn_lse_noncontig", "merge_out_bf16",
                                  "merge_lse_small", "merge_states_out_dtype", "compose_out_small",
                                  "norms_small", "norms_workspace_small", "contrib_workspace_small",
                                  "epsilon_eps_small"])
def test_binding_refuses_bad_outputs_before_calling(recorded, case):
    torch, rec, _ = recorded
    bf = torch.bfloat16
    q = torch.zeros(1, 2, 8, 64, dtype=bf)
    kv = torch.zeros(1, 2, 32, 64, dtype=bf)
    states, lses = torch.zeros(3, 16, 64), torch.zeros(3, 16)
    calls = {
        "attn_out_small": lambda: N.partition_attn(q, kv, kv, [(0, 32)], out=torch.zeros(1, 1, 2, 7, 64)),
        "attn_out_dtype": lambda: N.partition_attn(q, kv, kv, [(0, 32)], out=torch.zeros(1, 1, 2, 8, 64, dtype=bf)),
        "attn_lse_noncontig": lambda: N.partition_attn(q, kv, kv, [(0, 32)], lse=torch.zeros(1, 1, 8, 2).transpose(2, 3)),
        "merge_out_bf16": lambda: N.merge(list(states), list(lses), out=torch.zeros(16, 64, dtype=bf)),
        "merge_lse_small": lambda: N.merge(list(states), list(lses), lse=torch.zeros(15)),
        "merge_states_out_dtype": lambda: N.merge_states(list(states), list(lses), torch.float32,
                                                         out=torch.zeros(16, 64, dtype=bf)),
        "compose_out_small": lambda: N.compose_groups(states, lses, 2, out=torch.zeros(1, 16, 64)),
        "norms_small": lambda: N.state_norms(states.view(3, -1), norms=torch.zeros(2)),
        "norms_workspace_small": lambda: N.state_norms(states.view(3, -1), workspace=torch.zeros(8, dtype=torch.uint8)),
        "contrib_workspace_small": lambda: N.partition_contribution(lses, 8, workspace=torch.zeros(8, dtype=torch.uint8)),
        "epsilon_eps_small": lambda: N.planner_epsilon(torch.ones(4), torch.ones(4), 1, 2, 0.5, eps=torch.zeros(0)),
    }
    with pytest.raises(ValueError):
        calls[case]()
    assert rec.calls == [], "the library was called"


def test_binding_refuses_cpu_outputs():
    """With the real device check, a CPU output is refused like a CPU input (before any library call)."""
    import torch
    x = torch.zeros(2, 16, 64)
    with pytest.raises(ValueError, match="HIP device"):
        N.merge(list(x), list(torch.zeros(2, 16)))


def test_contribution_noalloc_rejects_sizes_beyond_its_scratch():
    """The allocation-free entry point holds AS_CONTRIBUTION_SCRATCH_BYTES of partial sums per device:
    larger score reductions are refused on the host, before any HIP call."""
    L = N.lib()
    P, rpg = 256, 256
    rows = rpg * 1025          # 1025 groups x 1 chunk x 256 partitions x 4 bytes > 1 MiB
    assert L.as_partition_contribution_workspace_size(P, rows, rpg) > N.CONTRIBUTION_SCRATCH_BYTES
    st = L.as_partition_contribution_noalloc(FAKE, P, rows, rpg, 0, 0x200000000, None)
    assert st == N.AS_ERR_INVALID_ARG and "scratch" in L.as_last_error().decode()
    st = L.as_partition_contribution_noalloc(FAKE, 0, rows, rpg, 0, FAKE, None)
    assert st == N.AS_ERR_INVALID_ARG
    # weights only need no scratch at all; nothing requested enqueues nothing
    assert L.as_partition_contribution_noalloc(FAKE, P, rows, rpg, 0, 0, None) == N.AS_OK
