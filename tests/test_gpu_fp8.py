"""GPU parity of the fp8 formats through the C ABI: fp8 E4M3 values (as_partition_attn_fp8_qkv,
grouped launches with fp8 v) and fp8 state payloads (E4M3 codes with one float32 factor per
row) written by a1 and read and written by as_merge_states and as_compose_groups.

Parity is against the fp64 oracle on the decoded values (oracle.fp8). Tolerances:
  - fp8 q/k/v: the bf16 tolerances (2e-2 on OUT, 1e-3 on LSE); the value codes are widened to
    bf16 exactly, so the only rounding beyond the fp8-q/k path is V's factor.
  - fp8 state payloads: the tolerance of the same state in fp32 plus the payload's own
    rounding: one E4M3 round-to-nearest-even of OUT * (448 / amax) is off by at most 2^-4 of
    its value (normal codes) or 2^-10 (subnormals), i.e. 2^-4 |OUT| + 2^-10 f in OUT units
    (f = amax / 448 the row's factor), plus a few fp32 roundings of the quotients (<= 2^-21 amax).
Where floating point decides a code, both sides decide it in fp32: the codes of a payload equal
torch's float8_e4m3fn rounding of the fp32 state that the same call computes (taken from the
fp32-state launch of the same inputs, whose arithmetic is the same up to the stores).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from sequence_dit_amd import _native as N
from sequence_dit_amd import inputs

pytestmark = pytest.mark.gpu

BF16_OUT, BF16_LSE, F32_TOL = 2e-2, 1e-3, 1e-5
DEV = "cuda:0"
FP8 = torch.float8_e4m3fn


def note(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


def dev(t):
    return t.to(DEV)


def dq(codes, scale):
    """Oracle decoding of fp8 codes [B, H, S, D] with per-(b, h) factors."""
    return oracle.fp8.dequantize(codes.cpu().view(torch.uint8).numpy(), scale.cpu().numpy())


def decode(st):
    """An Fp8States block decoded by the oracle: float64 [n, *shape]."""
    return oracle.fp8.decode_state(st.codes().cpu().numpy(), st.factors().cpu().numpy())


def quantize_rows(x):
    """The payload rule in fp32 (torch on the CPU): factor = amax / 448, codes = RNE E4M3 of
    clamp(x * (448 / amax)) per row of the last dimension; zero rows give codes 0, factor 0.
    Both quotients are tensor-by-tensor divisions (correctly rounded): torch evaluates a
    scalar-by-tensor quotient as a reciprocal times the scalar, two roundings."""
    x = x.float().cpu()
    amax = x.abs().amax(dim=-1)
    c448 = torch.full_like(amax, 448.0)
    qf = torch.where(amax > 0, c448 / torch.where(amax > 0, amax, c448), torch.zeros_like(amax))
    codes = (x * qf[..., None]).clamp(-448.0, 448.0).to(FP8).view(torch.uint8)
    return codes, amax / c448


def check_payload_rule(st, x32, what):
    """Codes and factors of an Fp8States block are the payload rule applied to the fp32 states x32."""
    codes, fac = quantize_rows(x32.reshape((st.n,) + st.shape))
    got_c, got_f = st.codes().cpu(), st.factors().cpu()
    nbad = int((got_c != codes.cpu()).sum())
    assert nbad == 0, f"{what}: {nbad} codes differ from the payload rule on the fp32 state"
    assert torch.equal(got_f.view(torch.int32), fac.cpu().view(torch.int32)), f"{what}: factors differ"


def check_decoded(st, lse, o_ref, l_ref, base_out, base_lse, what):
    """Decoded payloads against the oracle within the fp32-state tolerance plus the payload rounding."""
    got = decode(st).reshape(o_ref.shape)
    fac = st.factors().cpu().double().numpy().reshape(o_ref.shape[:-1])
    lse = lse.detach().cpu().double().numpy()
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf pattern differs"
    assert np.all(got[empty] == 0) and np.all(fac[empty] == 0), f"{what}: empty state payload is not 0"
    assert np.all(np.isfinite(got)), f"{what}: non-finite OUT"
    amax = fac * 448.0
    tol = (base_out + 2.0 ** -4 * (np.abs(o_ref) + base_out) * 1.001 + (2.0 ** -10 * fac + 2.0 ** -21 * amax)[..., None])
    excess = np.abs(got - o_ref) - tol
    assert np.all(excess <= 0), f"{what}: decoded OUT off by more than the bound (worst excess {excess.max():.3e})"
    el = np.abs(lse[~empty] - l_ref[~empty]).max() if (~empty).any() else 0.0
    assert el <= base_lse, f"{what}: LSE max-abs error {el:.3e} > {base_lse}"
    return np.abs(got - o_ref).max()


def check_states(out, lse, o_ref, l_ref, out_tol, lse_tol, what):
    out = out.detach().cpu().double().numpy()
    lse = lse.detach().cpu().double().numpy()
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf pattern differs"
    assert np.all(out[empty] == 0), f"{what}: empty state OUT is not 0"
    assert np.all(np.isfinite(out)), f"{what}: non-finite OUT"
    eo = np.abs(out - o_ref).max() if out.size else 0.0
    el = np.abs(lse[~empty] - l_ref[~empty]).max() if (~empty).any() else 0.0
    assert eo <= out_tol, f"{what}: OUT max-abs error {eo:.3e} > {out_tol}"
    assert el <= lse_tol, f"{what}: LSE max-abs error {el:.3e} > {lse_tol}"
    return eo, el


RAGGED = [(0, 200), (200, 201), (201, 201), (201, 777), (777, 1000), (100, 300), (0, 1000)]


# --------------------------------------------------------------------------- #
# fp8 values
# --------------------------------------------------------------------------- #

FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


@pytest.mark.parametrize("D", [128, 64])
def test_fp8_values_single_key_ranges_decode_every_code(D):
    """With one key per range, OUT is that key's V row times V's factor, exactly: every finite
    E4M3 code at every d position and byte lane, with factors 0.5 and -2 (powers of two keep the
    product exact). LSE is the fp8-q/k path's bit for bit (the score path is shared)."""
    B, H, Sq, Skv = 1, 2, 40, 256
    w = inputs.small_case_fp8(200 + D, B, H, Sq, Skv, D, [(0, 1)])
    j = np.arange(Skv)[:, None]
    d = np.arange(D)[None, :]
    v8 = np.stack([FINITE_CODES[(7 * j + 3 * d + 11 * h) % len(FINITE_CODES)] for h in range(H)])[None]
    v8t = torch.from_numpy(v8.copy()).view(FP8)
    v_scale = torch.tensor([[0.5, -2.0]], dtype=torch.float32)
    ranges = [(i, i + 1) for i in range(Skv)]
    note(f"fp8 values, single-key ranges D={D} P={len(ranges)}")
    out, lse = N.partition_attn_fp8_qkv(dev(w.q8), dev(w.k8), dev(v8t), dev(w.q_scale), dev(w.k_scale),
                                        dev(v_scale), ranges, w.scale)
    vb = torch.from_numpy(oracle.fp8.decode_e4m3(v8)).to(torch.bfloat16)   # exact: E4M3 values are bf16 values
    o2, l2 = N.partition_attn_fp8(dev(w.q8), dev(w.k8), dev(vb), dev(w.q_scale), dev(w.k_scale), ranges, w.scale)
    torch.cuda.synchronize()
    expect = dq(v8t, v_scale)                      # [B, H, Skv, D]
    expect = np.broadcast_to(np.transpose(expect, (2, 0, 1, 3))[:, :, :, None, :], out.shape)
    got = out.cpu().double().numpy()
    bad = int(np.sum(got != expect))
    assert bad == 0, f"{bad} OUT elements differ from decode(code) * factor"
    assert torch.equal(lse, l2), "LSE differs from the fp8-q/k path"


@pytest.mark.parametrize("state", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [128, 64])
def test_fp8_values_equal_bf16_values_path(D, state):
    """fp8 v with factor 1 is the fp8-q/k path on v's decoded values (bf16), bit for bit; both at
    parity with the oracle (the bf16 OUT tolerance taken at the values' scale: codes reach 448
    where the unit-variance values reach about 5)."""
    w = inputs.small_case_fp8(210 + D, 2, 3, 300, 1000, D, RAGGED)
    ones = torch.ones_like(w.v_scale)
    vb = torch.from_numpy(oracle.fp8.decode_e4m3(w.v8.view(torch.uint8).numpy())).to(torch.bfloat16)
    note(f"fp8 q/k/v vs fp8 q/k with decoded v D={D} state={state}")
    o8, l8 = N.partition_attn_fp8_qkv(dev(w.q8), dev(w.k8), dev(w.v8), dev(w.q_scale), dev(w.k_scale), dev(ones),
                                      w.ranges, w.scale, state)
    ob, lb = N.partition_attn_fp8(dev(w.q8), dev(w.k8), dev(vb), dev(w.q_scale), dev(w.k_scale), w.ranges, w.scale,
                                  state)
    torch.cuda.synchronize()
    assert torch.equal(o8, ob) and torch.equal(l8, lb), "fp8 v and its bf16 values give different states"
    o_ref, l_ref = oracle.partition_states(dq(w.q8, w.q_scale), dq(w.k8, w.k_scale), vb.double().numpy(),
                                           w.ranges, w.scale)
    vscale = float(vb.float().abs().max() / w.v.float().abs().max())
    check_states(o8.float(), l8, o_ref, l_ref, BF16_OUT * vscale, BF16_LSE, f"fp8 q/k/v D={D} {state}")


@pytest.mark.parametrize("D", [128, 64])
def test_fp8_qkv_small_ragged(D):
    """fp8 q, k, v with per-(b, h) factors (from the bf16 tensors) against the oracle on the decoded
    values: ragged, single-key, empty, overlapping and full ranges."""
    w = inputs.small_case_fp8(220 + D, 2, 3, 300, 1000, D, RAGGED)
    note(f"fp8 q/k/v small ragged D={D}")
    out, lse = N.partition_attn_fp8_qkv(dev(w.q8), dev(w.k8), dev(w.v8), dev(w.q_scale), dev(w.k_scale),
                                        dev(w.v_scale), w.ranges, w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(dq(w.q8, w.q_scale), dq(w.k8, w.k_scale), dq(w.v8, w.v_scale),
                                           w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"fp8 q/k/v D={D}")


def test_fp8_qkv_strided_views():
    """fp8 q/k/v as views with padded rows and an extra head (strides that are not the contiguous ones)."""
    B, H, Sq, Skv, D = 1, 2, 70, 333, 128
    w = inputs.small_case_fp8(230, B, H, Sq, Skv, D, [(0, 333), (5, 70), (300, 333)])
    qbig = torch.zeros((B, H, Sq + 16, D + 32), dtype=torch.uint8)
    qbig[:, :, 8:8 + Sq, :D] = w.q8.view(torch.uint8)
    kbig = torch.zeros((B, H + 1, Skv, D + 16), dtype=torch.uint8)
    kbig[:, 1:, :, :D] = w.k8.view(torch.uint8)
    vbig = torch.zeros((B, H + 1, Skv, D + 16), dtype=torch.uint8)
    vbig[:, 1:, :, :D] = w.v8.view(torch.uint8)
    qd = dev(qbig).view(FP8)[:, :, 8:8 + Sq, :D]
    kd = dev(kbig).view(FP8)[:, 1:, :, :D]
    vd = dev(vbig).view(FP8)[:, 1:, :, :D]
    note("fp8 q/k/v strided views")
    out, lse = N.partition_attn_fp8_qkv(qd, kd, vd, dev(w.q_scale), dev(w.k_scale), dev(w.v_scale), w.ranges,
                                        w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(dq(w.q8, w.q_scale), dq(w.k8, w.k_scale), dq(w.v8, w.v_scale),
                                           w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, "fp8 q/k/v strided")


RANGES_G = [(0, 200), (200, 201), (201, 201), (201, 777), (777, 1000), (100, 300), (0, 1000), (5, 5), (333, 334)]
STARTS_G = [0, 3, 3, 5, 9]


@pytest.mark.parametrize("D", [128, 64])
def test_grouped_fp8_values(D):
    """Grouped launches with fp8 q/k/v: every group's composed state and every partition's LSE, and
    a state folded into group 0."""
    w = inputs.small_case_fp8(240 + D, 2, 3, 300, 1000, D, RANGES_G)
    g = np.random.default_rng(D)
    fo = g.standard_normal((2, 3, 300, D)).astype(np.float32)
    fl = (g.standard_normal((2, 3, 300)) * 2 + 4).astype(np.float32)
    note(f"grouped fp8 q/k/v D={D} groups={STARTS_G}")
    out, lse, plse = N.partition_attn_grouped(dev(w.q8), dev(w.k8), dev(w.v8), w.ranges, STARTS_G, w.scale,
                                              fold=(dev(torch.from_numpy(fo)), dev(torch.from_numpy(fl))),
                                              q_scale=dev(w.q_scale), k_scale=dev(w.k_scale),
                                              v_scale=dev(w.v_scale))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(dq(w.q8, w.q_scale), dq(w.k8, w.k_scale), dq(w.v8, w.v_scale),
                                           w.ranges, w.scale)
    got = plse.cpu().double().numpy()
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(got), ~fin)
    assert np.abs(got[fin] - l_ref[fin]).max() <= BF16_LSE
    for gi in range(len(STARTS_G) - 1):
        s, e = STARTS_G[gi], STARTS_G[gi + 1]
        os_, ls_ = list(o_ref[s:e]), list(l_ref[s:e])
        if gi == 0:
            os_.append(fo.astype(np.float64))
            ls_.append(fl.astype(np.float64))
        if os_:
            ro, rl = oracle.merge(np.stack(os_), np.stack(ls_))
        else:
            ro, rl = np.zeros(o_ref.shape[1:]), np.full(l_ref.shape[1:], -np.inf)
        check_states(out[gi], lse[gi], ro, rl, BF16_OUT, BF16_LSE, f"grouped fp8 q/k/v group {gi}")


# --------------------------------------------------------------------------- #
# fp8 state payloads written by a1
# --------------------------------------------------------------------------- #

def run_attn(path, w, state):
    if path == "bf16":
        return N.partition_attn_states(dev(w.q), dev(w.k), dev(w.v), w.ranges, w.scale, state)
    if path == "fp8qk":
        return N.partition_attn_fp8(dev(w.q8), dev(w.k8), dev(w.v), dev(w.q_scale), dev(w.k_scale), w.ranges,
                                    w.scale, state)
    return N.partition_attn_fp8_qkv(dev(w.q8), dev(w.k8), dev(w.v8), dev(w.q_scale), dev(w.k_scale),
                                    dev(w.v_scale), w.ranges, w.scale, state)


def oracle_for(path, w):
    if path == "bf16":
        return oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    v = w.v if path == "fp8qk" else dq(w.v8, w.v_scale)
    return oracle.partition_states(dq(w.q8, w.q_scale), dq(w.k8, w.k_scale), v, w.ranges, w.scale)


@pytest.mark.parametrize("path", ["bf16", "fp8qk", "fp8qkv"])
@pytest.mark.parametrize("D", [128, 64])
def test_attention_writes_fp8_state_payloads(D, path):
    """a1 with fp8 state payloads: LSE bit for bit the fp32-state launch's, codes and factors the
    payload rule on that launch's fp32 OUT, decoded OUT within the bound of the oracle; empty
    partitions give codes 0 and factor 0."""
    w = inputs.small_case_fp8(250 + D, 2, 3, 300, 1000, D, RAGGED)
    note(f"fp8 state payloads from a1 D={D} path={path}")
    st, l8 = run_attn(path, w, FP8)
    o32, l32 = run_attn(path, w, torch.float32)
    torch.cuda.synchronize()
    assert isinstance(st, N.Fp8States) and st.n == len(RAGGED) and st.shape == (2, 3, 300, D)
    assert torch.equal(l8, l32), "LSE differs from the fp32-state launch"
    check_payload_rule(st, o32, f"a1 payload D={D} {path}")
    o_ref, l_ref = oracle_for(path, w)
    err = check_decoded(st, l8, o_ref, l_ref, BF16_OUT, BF16_LSE, f"a1 payload D={D} {path}")
    note(f"a1 fp8 payload D={D} {path}: decoded OUT max-abs {err:.3e}")


# --------------------------------------------------------------------------- #
# fp8 state payloads in composition
# --------------------------------------------------------------------------- #

def fp8_block(codes, factors, shape=None):
    """An Fp8States block on the device holding the given codes [n, rows, D] and factors [n, rows]."""
    n, rows, D = codes.shape
    st = N.Fp8States.empty(n, shape or (rows, D), DEV)
    st.codes().copy_(dev(torch.from_numpy(codes.reshape((n,) + st.shape))))
    st.factors().copy_(dev(torch.from_numpy(factors.reshape((n,) + st.shape[:-1]))))
    return st


def random_states(seed, n, rows, D, n_empty=0):
    g = np.random.default_rng(seed)
    outs = g.standard_normal((n, rows, D)).astype(np.float32)
    lses = (g.standard_normal((n, rows)) * 4).astype(np.float32)
    if n_empty:
        idx = g.choice(n * rows, size=n_empty, replace=False)
        outs.reshape(n * rows, D)[idx] = 0
        lses.reshape(-1)[idx] = -np.inf
    return outs, lses


def make_inputs(kind, seed, n, rows, D, n_empty):
    """(device inputs as a list of single states, their decoded/stored values [n, rows, D], LSE)."""
    if kind == FP8:
        codes, fac, lses = inputs.random_fp8_states(seed, n, rows, D, n_empty)
        codes[:, 0] = 0
        fac[:, 0] = 0
        lses[:, 0] = -np.inf
        st = fp8_block(codes, fac)
        return [st[i] for i in range(n)], oracle.fp8.decode_state(codes, fac), lses, st
    outs, lses = random_states(seed, n, rows, D, n_empty)
    outs[:, 0] = 0
    lses[:, 0] = -np.inf
    od = dev(torch.from_numpy(outs)).to(kind)
    return list(od), od.double().cpu().numpy(), lses, od


def check_composed(out, lse, r_out, r_lse, out_dt, what):
    if out_dt == FP8:
        check_decoded(out, lse, r_out, r_lse, F32_TOL, F32_TOL, what)
    elif out_dt == torch.float32:
        check_states(out, lse, r_out, r_lse, F32_TOL, F32_TOL, what)
    else:
        got = out.float().cpu().double().numpy()
        err = np.abs(got - r_out) - (np.abs(r_out) * 2.0 ** -8 + 1e-5)
        assert np.all(err <= 0), f"{what}: off by more than a bf16 rounding (worst excess {err.max():.3e})"
        fin = np.isfinite(r_lse)
        assert np.abs(lse.cpu().double().numpy()[fin] - r_lse[fin]).max() <= F32_TOL


MERGE_CASES = [(28, 300, 128, FP8, torch.float32), (5, 777, 128, FP8, FP8), (32, 129, 64, torch.float32, FP8),
               (9, 301, 32, FP8, torch.bfloat16), (64, 33, 256, torch.bfloat16, FP8), (3, 50, 64, FP8, FP8),
               (1, 20, 128, FP8, FP8)]


@pytest.mark.parametrize("n,rows,D,in_dt,out_dt", MERGE_CASES, ids=lambda x: str(x).replace("torch.", ""))
def test_merge_states_fp8_matches_oracle(n, rows, D, in_dt, out_dt):
    """as_merge_states reading and/or writing fp8 payloads against the oracle's merge of the decoded
    (or stored) inputs; an fp8 output's codes follow the payload rule on the fp32-output merge."""
    ins, vals, lses, _ = make_inputs(in_dt, n * 11 + D, n, rows, D, rows // 3)
    ld = dev(torch.from_numpy(lses))
    note(f"merge_states n={n} rows={rows} D={D} {in_dt}->{out_dt}")
    m_out, m_lse = N.merge_states(ins, list(ld), out_dt)
    torch.cuda.synchronize()
    r_out, r_lse = oracle.merge(vals, lses)
    check_composed(m_out, m_lse, r_out, r_lse, out_dt, f"merge_states {in_dt}->{out_dt}")
    if out_dt == FP8:
        f_out, f_lse = N.merge_states(ins, list(ld), torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(f_lse, m_lse)
        check_payload_rule(m_out, f_out, f"merge_states fp8 OUT n={n}")


def test_merge_fp8_single_state_is_its_decoded_values():
    """One fp8 state composed with empty ones gives fl32(factor * decode(code)) bit for bit (the
    factor meets the code in one fp32 product) and its LSE unchanged."""
    codes, fac, lses = inputs.random_fp8_states(3, 1, 257, 128)
    st = fp8_block(codes, fac)
    e = N.Fp8States.empty(1, (257, 128), DEV)
    e.data.zero_()
    x_lse = dev(torch.from_numpy(lses[0]))
    e_lse = torch.full_like(x_lse, float("-inf"))
    note("fp8 merge identity")
    m_out, m_lse = N.merge_states([e, st[0], e], [e_lse, x_lse, e_lse], torch.float32)
    torch.cuda.synchronize()
    vals = torch.from_numpy(oracle.fp8.decode_e4m3(codes[0])).float() * torch.from_numpy(fac[0])[:, None]
    assert torch.equal(m_out.cpu().view(torch.int32), vals.view(torch.int32))
    assert torch.equal(m_lse, x_lse)


COMPOSE_CASES = [(32, 4, 300, 128, FP8, FP8), (7, 3, 129, 64, torch.float32, FP8), (32, 8, 384, 128, FP8,
                 torch.float32), (6, 1, 50, 32, FP8, torch.bfloat16), (5, 64, 33, 256, FP8, FP8)]


@pytest.mark.parametrize("P,group,rows,D,in_dt,out_dt", COMPOSE_CASES, ids=lambda x: str(x).replace("torch.", ""))
def test_compose_groups_fp8_matches_oracle(P, group, rows, D, in_dt, out_dt):
    """Group-wise composition of fp8 payload blocks (and into them) against the oracle; one launch
    over all groups equals the per-group merges bit for bit."""
    _, vals, lses, block = make_inputs(in_dt, P * 5 + group, P, rows, D, rows // 2)
    ld = dev(torch.from_numpy(lses))
    note(f"compose_groups P={P} group={group} rows={rows} D={D} {in_dt}->{out_dt}")
    g_out, g_lse = N.compose_groups(block, ld, group, out_dt)
    torch.cuda.synchronize()
    r_out, r_lse = oracle.compose_groups(vals, lses, group)
    G = (P + group - 1) // group
    assert (g_out.n if out_dt == FP8 else g_out.shape[0]) == G
    check_composed(g_out, g_lse, r_out, r_lse, out_dt, f"compose_groups {in_dt}->{out_dt}")
    for k in range(0, P, max(1, P // 4 // group) * group):
        ins = [block[i] for i in range(k, min(k + group, P))]
        m_out, m_lse = N.merge_states(ins, list(ld[k:k + group]), out_dt)
        torch.cuda.synchronize()
        if out_dt == FP8:   # (the payloads' padding bytes are not written)
            assert torch.equal(m_out.codes(), g_out[k // group].codes()), k
            assert torch.equal(m_out.factors().view(torch.int32), g_out[k // group].factors().view(torch.int32)), k
        else:
            assert torch.equal(m_out, g_out[k // group]), k
        assert torch.equal(m_lse, g_lse[k // group]), k


def test_fp8_payload_roundtrip_through_attention_and_compose():
    """a1 writes fp8 payloads, compose_groups reads them: the composed states match the oracle's
    composition of the decoded payloads (the composition adds no error beyond fp32)."""
    w = inputs.small_case_fp8(260, 1, 3, 300, 1200, 128, inputs.equal_ranges(1200, 8))
    note("fp8 payloads: a1 -> compose_groups")
    st, lse = N.partition_attn_fp8_qkv(dev(w.q8), dev(w.k8), dev(w.v8), dev(w.q_scale), dev(w.k_scale),
                                       dev(w.v_scale), w.ranges, w.scale, FP8)
    g_out, g_lse = N.compose_groups(st, lse, 4, torch.float32)
    torch.cuda.synchronize()
    vals = decode(st).reshape(8, -1, 128)
    r_out, r_lse = oracle.compose_groups(vals, lse.cpu().double().numpy().reshape(8, -1), 4)
    check_states(g_out.reshape(2, -1, 128), g_lse.reshape(2, -1), r_out, r_lse, F32_TOL, F32_TOL, "a1 -> compose")


# --------------------------------------------------------------------------- #
# full size
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("cfg", [2, 3])
def test_fp8_qkv_full_size_image_and_video_payloads(cfg):
    """The image and video DiT workloads at full size with fp8 q/k/v and fp8 state payloads, every
    element, in the launch configuration of the benchmark."""
    w = inputs.with_fp8(inputs.make(cfg))
    note(f"fp8 q/k/v full size {w.name}, fp8 payloads")
    st, lse = N.partition_attn_fp8_qkv(dev(w.q8), dev(w.k8), dev(w.v8), dev(w.q_scale), dev(w.k_scale),
                                       dev(w.v_scale), w.ranges, w.scale, FP8)
    o32, l32 = N.partition_attn_fp8_qkv(dev(w.q8), dev(w.k8), dev(w.v8), dev(w.q_scale), dev(w.k_scale),
                                        dev(w.v_scale), w.ranges, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(lse, l32)
    check_payload_rule(st, o32, f"config {cfg} payload")
    o_ref, l_ref = oracle.partition_states(dq(w.q8, w.q_scale), dq(w.k8, w.k_scale), dq(w.v8, w.v_scale),
                                           w.ranges, w.scale)
    eo, el = check_states(o32, l32, o_ref, l_ref, BF16_OUT, BF16_LSE, f"config {cfg} fp8 q/k/v")
    err = check_decoded(st, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"config {cfg} payload")
    note(f"config {cfg} fp8 q/k/v: OUT max-abs {eo:.3e}, LSE {el:.3e}, decoded payload {err:.3e}")
