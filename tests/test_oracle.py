"""Pins for the fp64 oracle: library routines, closed forms, invariants, a hand-worked example.

Each ``check_*`` takes the oracle module so that ``test_pins_catch_planted_mistakes``
can run the same checks against copies of the oracle with a mistake planted in
the source (on the CPU) and confirm that some check fails for each mistake.
"""
import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from sequence_dit_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_states.txt")
GOLDEN_PLANNER = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_planner.txt")


def rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa(q, k, v, scale):
    """torch's reference scaled-dot-product attention in float64 on the CPU."""
    t = lambda x: torch.as_tensor(np.asarray(x, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale).numpy()


def torch_lse(q, k, scale):
    t = lambda x: torch.as_tensor(np.asarray(x, dtype=np.float64))
    return torch.logsumexp(scale * (t(q) @ t(k).transpose(-1, -2)), dim=-1).numpy()


# --------------------------------------------------------------------------- #
# Golden fixture parsing
# --------------------------------------------------------------------------- #

def parse_value(s):
    s = s.strip()
    if s == "-inf":
        return -math.inf
    if s.startswith("ln(") and s.endswith(")"):
        return math.log(Fraction(s[3:-1]))
    if s.startswith("sqrt(") and s.endswith(")"):
        return math.sqrt(Fraction(s[5:-1]))
    return float(Fraction(s))


def load_golden(path=GOLDEN):
    data = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        name, rest = line.split(":", 1)
        rows = [[parse_value(x) for x in r.split(",")] for r in rest.split(";")]
        data[name.strip()] = rows
    return data


# --------------------------------------------------------------------------- #
# Pins (each takes the oracle module)
# --------------------------------------------------------------------------- #

RAGGED = [(0, 5), (5, 6), (6, 6), (6, 17), (17, 23)]  # regular, single key, empty, ragged


def check_golden(orc):
    g = load_golden()
    q = np.array(g["q"])[None, None]            # [1,1,1,2]
    k = np.array(g["k"])[None, None]            # [1,1,4,2]
    v = np.array(g["v"])[None, None]
    ranges = [tuple(int(x) for x in r) for r in g["ranges"]]
    scale = g["scale"][0][0]
    out, lse = orc.partition_states(q, k, v, ranges, scale)
    np.testing.assert_allclose(out[:, 0, 0, 0], np.array(g["out"]), rtol=0, atol=1e-14)
    want_lse = np.array(g["lse"])[:, 0]
    assert np.isneginf(lse[2, 0, 0, 0]) and np.isneginf(want_lse[2])
    np.testing.assert_allclose(lse[:2, 0, 0, 0], want_lse[:2], rtol=0, atol=1e-14)
    m_out, m_lse = orc.merge(out, lse)
    np.testing.assert_allclose(m_out[0, 0, 0], np.array(g["merged_out"][0]), rtol=0, atol=1e-14)
    assert abs(m_lse[0, 0, 0] - g["merged_lse"][0][0]) < 1e-14
    w, scores = orc.contribution(lse.reshape(3, 1), 1)
    np.testing.assert_allclose(w[:, 0], np.array(g["weights"])[:, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(scores[0], np.array(g["weights"])[:, 0], rtol=0, atol=1e-14)


def check_bruteforce_loops(orc):
    """Pure-Python loops (math.exp) on a tiny case, independent of numpy."""
    q, k, v = rand(1, 2, 3), rand(2, 5, 3), rand(3, 5, 4)  # Sq=2, Skv=5, D=3, Dv=4
    scale = 0.7
    ranges = [(0, 2), (2, 5)]
    out, lse = orc.partition_states(q[None, None], k[None, None], v[None, None], ranges, scale)
    for i, (s, e) in enumerate(ranges):
        for r in range(2):
            z = [scale * sum(q[r, d] * k[j, d] for d in range(3)) for j in range(s, e)]
            tot = sum(math.exp(x) for x in z)
            assert abs(lse[i, 0, 0, r] - math.log(tot)) < 1e-12
            for c in range(4):
                o = sum(math.exp(z[j - s]) / tot * v[j, c] for j in range(s, e))
                assert abs(out[i, 0, 0, r, c] - o) < 1e-12


def check_states_vs_sdpa(orc):
    """Each partition state is torch SDPA / logsumexp over that partition's keys."""
    B, H, Sq, Skv, D = 2, 3, 7, 23, 8
    q, k, v = rand(10, B, H, Sq, D), rand(11, B, H, Skv, D), rand(12, B, H, Skv, D)
    scale = D ** -0.5
    out, lse = orc.partition_states(q, k, v, RAGGED, scale)
    assert out.shape == (len(RAGGED), B, H, Sq, D) and lse.shape == (len(RAGGED), B, H, Sq)
    for i, (s, e) in enumerate(RAGGED):
        if e == s:
            assert np.all(out[i] == 0) and np.all(np.isneginf(lse[i]))
            continue
        np.testing.assert_allclose(out[i], sdpa(q, k[:, :, s:e], v[:, :, s:e], scale), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[i], torch_lse(q, k[:, :, s:e], scale), rtol=0, atol=1e-12)


def check_merge_equals_full(orc):
    """Composing the states of disjoint ranges that cover all keys gives full attention."""
    B, H, Sq, Skv, D = 1, 2, 9, 23, 16
    q, k, v = rand(20, B, H, Sq, D), rand(21, B, H, Skv, D), rand(22, B, H, Skv, D)
    scale = D ** -0.5
    out, lse = orc.partition_states(q, k, v, RAGGED, scale)
    m_out, m_lse = orc.merge(out, lse)
    np.testing.assert_allclose(m_out, sdpa(q, k, v, scale), rtol=0, atol=1e-12)
    np.testing.assert_allclose(m_lse, torch_lse(q, k, scale), rtol=0, atol=1e-12)
    f_out, f_lse = orc.full_attention(q, k, v, scale)
    np.testing.assert_allclose(f_out, m_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(f_lse, m_lse, rtol=0, atol=1e-12)


def check_identity_bitexact(orc):
    """Composing with the empty state (0, -inf) returns the other state bit for bit."""
    o = rand(30, 6, 5) * 3
    l = rand(31, 6) * 10
    e_o, e_l = np.zeros_like(o), np.full_like(l, -np.inf)
    for a, b in (((o, l), (e_o, e_l)), ((e_o, e_l), (o, l))):
        r_o, r_l = orc.merge_pair(a, b)
        assert np.array_equal(r_o, o) and np.array_equal(r_l, l)
    r_o, r_l = orc.merge(np.stack([e_o, o, e_o]), np.stack([e_l, l, e_l]))
    assert np.array_equal(r_o, o) and np.array_equal(r_l, l)
    # only empty inputs: the empty state, no NaN
    r_o, r_l = orc.merge(np.stack([e_o, e_o]), np.stack([e_l, e_l]))
    assert np.all(r_o == 0) and np.all(np.isneginf(r_l))


def check_closed_forms(orc):
    D, scale = 8, 0.3
    q, k, v = rand(40, 1, 1, 3, D), rand(41, 1, 1, 6, D), rand(42, 1, 1, 6, D)
    # single key: LSE = scale*<q,k>, OUT = v
    out, lse = orc.partition_states(q, k, v, [(2, 3)], scale)
    np.testing.assert_allclose(lse[0, 0, 0], scale * q[0, 0] @ k[0, 0, 2], rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[0, 0, 0], np.broadcast_to(v[0, 0, 2], (3, D)), rtol=0, atol=1e-13)
    # Q = 0: LSE = ln n, OUT = mean of the partition's values
    out, lse = orc.partition_states(np.zeros_like(q), k, v, [(0, 4), (4, 6)], scale)
    np.testing.assert_allclose(lse[:, 0, 0, 0], [math.log(4), math.log(2)], rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[0, 0, 0, 1], v[0, 0, :4].mean(0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[1, 0, 0, 2], v[0, 0, 4:].mean(0), rtol=0, atol=1e-13)
    # identical keys: LSE = scale*<q,k> + ln n, OUT = mean of values
    kk = np.broadcast_to(k[:, :, :1], k.shape).copy()
    out, lse = orc.partition_states(q, kk, v, [(0, 5)], scale)
    np.testing.assert_allclose(lse[0, 0, 0], scale * q[0, 0] @ k[0, 0, 0] + math.log(5), rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[0, 0, 0, 0], v[0, 0, :5].mean(0), rtol=0, atol=1e-13)
    # equal-LSE pair: LSE + ln 2, mean of OUTs
    a_o, b_o, l = rand(43, 4, D), rand(44, 4, D), rand(45, 4)
    r_o, r_l = orc.merge_pair((a_o, l), (b_o, l))
    np.testing.assert_allclose(r_l, l + math.log(2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(r_o, (a_o + b_o) / 2, rtol=0, atol=1e-13)
    # shifting every LSE by c shifts the result by c and keeps OUT
    outs, lses = rand(46, 5, 4, D), rand(47, 5, 4)
    r0 = orc.merge(outs, lses)
    r1 = orc.merge(outs, lses + 7.5)
    np.testing.assert_allclose(r1[1], r0[1] + 7.5, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r1[0], r0[0], rtol=0, atol=1e-12)


def check_contribution(orc):
    B, H, Sq, Skv, D = 1, 2, 5, 23, 8
    q, k, v = rand(50, B, H, Sq, D), rand(51, B, H, Skv, D), rand(52, B, H, Skv, D)
    scale = D ** -0.5
    P = len(RAGGED)
    out, lse = orc.partition_states(q, k, v, RAGGED, scale)
    w, scores = orc.contribution(lse.reshape(P, -1), Sq)
    assert w.shape == (P, B * H * Sq) and scores.shape == (B * H, P)
    np.testing.assert_allclose(w.sum(0), 1.0, rtol=0, atol=1e-13)
    # w_i = attention mass that full softmax puts on partition i (torch softmax)
    t = lambda x: torch.as_tensor(x)
    prob = torch.softmax(scale * (t(q) @ t(k).transpose(-1, -2)), dim=-1).numpy()
    for i, (s, e) in enumerate(RAGGED):
        np.testing.assert_allclose(w[i], prob[..., s:e].sum(-1).reshape(-1), rtol=0, atol=1e-13)
    # Q = 0: w_i = n_i / Skv
    _, lse0 = orc.partition_states(np.zeros_like(q), k, v, RAGGED, scale)
    w0, s0 = orc.contribution(lse0.reshape(P, -1), Sq)
    n = np.array([e - s for s, e in RAGGED], dtype=float)
    np.testing.assert_allclose(w0, np.broadcast_to((n / Skv)[:, None], w0.shape), rtol=0, atol=1e-14)
    np.testing.assert_allclose(s0, np.broadcast_to(n / Skv, s0.shape), rtol=0, atol=1e-14)
    # groups of one row give w itself; one group gives the column means
    _, s1 = orc.contribution(lse.reshape(P, -1), 1)
    np.testing.assert_allclose(s1, w.T, rtol=0, atol=1e-15)
    _, sall = orc.contribution(lse.reshape(P, -1), B * H * Sq)
    np.testing.assert_allclose(sall[0], w.sum(1) / (B * H * Sq), rtol=0, atol=1e-14)


def check_reuse(orc):
    w = inputs.small_case(3, 1, 2, 6, 40, 8, [(0, 10), (10, 20), (20, 30), (30, 40)], dtype=torch.float32)
    near = orc.nearest_partitions(4, 1, 2)
    assert near == [0, 1]
    o, l = orc.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    # zero residual: reuse equals full attention
    r_o, r_l, _, _ = orc.selective_reuse(o, l, o, l, near)
    f_o, f_l = orc.full_attention(w.q, w.k, w.v, w.scale)
    np.testing.assert_allclose(r_o, f_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r_l, f_l, rtol=0, atol=1e-12)
    # error grows with the residual between the steps
    errs = []
    for res in (0.0, 0.01, 0.05):
        g = np.random.default_rng(99)
        q1, k1, v1 = (x.double().numpy() + res * g.standard_normal(x.shape) for x in (w.q, w.k, w.v))
        o1, l1 = orc.partition_states(q1, k1, v1, w.ranges, w.scale)
        r_o, _, _, _ = orc.selective_reuse(o, l, o1, l1, near)
        errs.append(orc.mse(r_o, orc.full_attention(q1, k1, v1, w.scale)[0]))
    assert errs[0] < 1e-25 < errs[1] < errs[2]


def check_mse(orc):
    """The reported error measure: hand-worked value (golden file), a 3-d layout of the same
    numbers, and the zero of identical inputs."""
    g = load_golden()
    a, b = np.array(g["mse_a"]), np.array(g["mse_b"])
    assert orc.mse(a, b) == g["mse"][0][0]
    assert orc.mse(a.reshape(2, 1, 2), b.reshape(2, 1, 2)) == g["mse"][0][0]
    assert orc.mse(b, a) == g["mse"][0][0]
    assert orc.mse(a, a) == 0.0


def check_compose_groups(orc):
    g = np.random.default_rng(21)
    P, rows, D = 7, 5, 3
    outs = g.standard_normal((P, rows, D))
    lses = g.standard_normal((P, rows)) * 4
    outs[5], lses[5] = 0.0, -np.inf            # one empty partition
    full_o, full_l = orc.merge(outs, lses)
    # groups of one: the states themselves, bit for bit
    o1, l1 = orc.compose_groups(outs, lses, 1)
    assert np.array_equal(o1, outs) and np.array_equal(l1, lses)
    for group in (2, 3, 4, 7, 9):
        go, gl = orc.compose_groups(outs, lses, group)
        assert go.shape == ((P + group - 1) // group, rows, D)
        # composing the group states again gives the composition of all of them
        mo, ml = orc.merge(go, gl)
        np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)
        # the last group holds exactly the last partitions
        k = (P - 1) // group
        lo, ll = orc.merge(outs[k * group:], lses[k * group:])
        np.testing.assert_allclose(go[-1], lo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(gl[-1], ll, rtol=0, atol=1e-12)
    # a group made only of empty states is the empty state
    e_o, e_l = orc.compose_groups(np.zeros((2, rows, D)), np.full((2, rows), -np.inf), 2)
    assert np.all(e_o == 0) and np.all(np.isneginf(e_l))


# --------------------------------------------------------------------------- #
# Planner statistics (Eqs. 9, 10, 12, 13, Algorithm 1)
# --------------------------------------------------------------------------- #

def check_planner_golden(orc):
    g = load_golden(GOLDEN_PLANNER)
    pl = orc.planner
    a = np.array(g["norm_a"]).reshape(2, 2, 2)
    b = np.array(g["norm_b"]).reshape(2, 2, 2)
    np.testing.assert_allclose(pl.state_norm(a), g["norm_a_expected"][0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(pl.state_norm(a, b), g["norm_diff_expected"][0], rtol=0, atol=1e-15)
    local, group = int(g["plan_params"][0][0]), int(g["plan_params"][0][1])
    eps, eps_local = g["plan_params"][0][2], g["plan_params"][0][3]
    r = pl.planner(g["plan_norms"][0], g["plan_drift"][0][0], g["plan_weights"][0], local, group, eps, eps_local)
    for key in ("alpha", "delta", "ase"):
        np.testing.assert_allclose(r[key], g["plan_" + key][0], rtol=0, atol=1e-15)
    assert list(r["compute"]) == [int(x) for x in g["plan_compute"][0]]
    assert int(r["anchor"]) == int(g["plan_anchor"][0][0])
    for frac, want in g["eps_cases"]:
        got = pl.epsilon(g["eps_corr"][0], g["plan_weights"][0], local, group, frac)
        assert (got == want) if math.isinf(want) else abs(got - want) < 1e-15, (frac, got, want)


def check_norms(orc):
    pl = orc.planner
    a = rand(41, 3, 2, 5)
    b = rand(42, 3, 2, 5)
    # pure-Python loops
    for mode in (None, b):
        got = pl.state_norm(a, mode)
        for i in range(3):
            acc = 0.0
            for r in range(2):
                for c in range(5):
                    d = a[i, r, c] - (0.0 if mode is None else mode[i, r, c])
                    acc += d * d
            assert abs(got[i] - math.sqrt(acc)) < 1e-12
    # homogeneity, zero difference, disjoint supports (Pythagoras)
    np.testing.assert_allclose(pl.state_norm(-3 * a), 3 * pl.state_norm(a), rtol=1e-14)
    np.testing.assert_array_equal(pl.state_norm(a, a), np.zeros(3))
    lo, hi = a.copy(), a.copy()
    lo[:, :, 3:] = 0
    hi[:, :, :3] = 0
    np.testing.assert_allclose(pl.state_norm(a) ** 2, pl.state_norm(lo) ** 2 + pl.state_norm(hi) ** 2, rtol=1e-13)
    np.testing.assert_allclose(pl.state_norm(lo, -hi), pl.state_norm(a), rtol=1e-14)


def check_planner_invariants(orc):
    pl = orc.planner
    g = np.random.default_rng(5)
    P, group = 11, 3                      # groups {0,1,2} {3,4,5} {6,7,8} {9,10}
    norms = g.uniform(0.5, 4, P)
    w = g.dirichlet(np.ones(P))
    for local in (0, 4, 10):
        alpha = pl.scale_ratios(norms, local)
        assert alpha[local] == 1.0
        np.testing.assert_allclose(pl.scale_ratios(7.5 * norms, local), alpha, rtol=1e-15)
        np.testing.assert_allclose(alpha * norms[local], norms, rtol=1e-15)
        d1 = pl.drift_errors(alpha, 0.3)
        np.testing.assert_allclose(pl.drift_errors(alpha, 0.6), 2 * d1, rtol=1e-15)
        np.testing.assert_allclose(d1[local], 0.3, rtol=1e-15)
        ase = pl.group_errors(w, d1, group)
        assert len(ase) == 4
        np.testing.assert_allclose(ase[3], w[9] * d1[9] + w[10] * d1[10], rtol=1e-15)
        np.testing.assert_allclose(ase.sum(), np.dot(w, d1), rtol=1e-14)
        # raising one weight raises exactly its group's error
        w2 = w.copy()
        w2[7] += 0.5
        diff = pl.group_errors(w2, d1, group) - ase
        assert diff[2] > 0 and np.all(diff[[0, 1, 3]] == 0)
        # no drift: every non-local group is reused; -inf threshold: everything computed
        z = pl.planner(norms, 0.0, w, local, group, 0.0, 1.0)
        assert np.all(z["ase"] == 0) and list(z["compute"]) == [int(k == local // group) for k in range(4)]
        assert not z["anchor"] and pl.planner(norms, 2.0, w, local, group, 0.0, 1.0)["anchor"]
        assert list(pl.decide(ase, local, group, -math.inf)) == [1, 1, 1, 1]
        # a threshold between two errors splits the non-local groups by their error
        c = pl.decide(ase, local, group, float(np.median(ase)))
        for k in range(4):
            assert c[k] == (1 if k == local // group else int(ase[k] > np.median(ase)))


def check_epsilon(orc):
    pl = orc.planner
    g = np.random.default_rng(9)
    P, group, local = 32, 4, 16            # 8 groups, local group 4, G' = 7
    corr = g.uniform(0, 1, P)
    w = g.dirichlet(np.ones(P))
    E = pl.group_errors(w, corr, group)
    others = np.delete(E, local // group)
    prev = -math.inf
    for R in (0.0, 0.1, 0.15, 1 / 7, 0.3, 0.5, 0.75, 0.99, 1.0):
        eps = pl.epsilon(corr, w, local, group, R)
        m = int(np.floor(np.float32(R) * np.float32(7)))
        assert int(np.sum(others <= eps)) == m, (R, eps)
        assert eps >= prev
        prev = eps
        if m:
            assert eps in list(others)
        # planning with the threshold on the correction errors reuses exactly m groups
        c = pl.decide(E, local, group, eps)
        assert c[local // group] == 1 and int(np.sum(c == 0)) == m
    assert pl.epsilon(corr, w, local, group, 1.0) == others.max()
    assert pl.epsilon(corr, w, local, group, 0.0) == -math.inf


FP8_HAND = {  # E4M3 codes worked by hand: sign | exponent (bias 7) | mantissa
    0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x39: 1.125, 0x40: 2.0, 0x30: 0.5, 0x77: 240.0, 0x7E: 448.0,
    0xFE: -448.0, 0x08: 2.0 ** -6, 0x07: 7 / 8 * 2.0 ** -6, 0x01: 2.0 ** -9, 0x81: -(2.0 ** -9)}


def check_fp8(orc):
    """E4M3 decoding: hand-worked codes, the NaN codes, torch's own float8_e4m3fn
    conversion on all 256 codes (library routine), strict monotonicity of the
    positive codes, and per-(b, h) dequantisation on a brute-force loop."""
    dec = orc.fp8.decode_e4m3
    for c, v in FP8_HAND.items():
        assert dec(np.array([c]))[0] == v, (hex(c), dec(np.array([c]))[0], v)
    assert np.isnan(dec(np.array([0x7F, 0xFF]))).all()
    codes = np.arange(256, dtype=np.uint8)
    mine = dec(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.all(np.diff(mine[:127]) > 0)
    g = np.random.default_rng(5)
    cq = g.integers(0, 256, size=(2, 3, 4, 5)).astype(np.uint8)
    cq[cq & 0x7F == 0x7F] = 0x38
    sc = np.array([[0.5, 2.0, 3.0], [1.0, 0.25, 7.0]])
    got = orc.fp8.dequantize(cq, sc)
    for b in range(2):
        for h in range(3):
            for i in range(4):
                for j in range(5):
                    assert got[b, h, i, j] == FP8_ALL[int(cq[b, h, i, j])] * sc[b, h]
    # fp8 states: one factor per row (rows != D, so a factor taken per column fails)
    fr = np.array([[0.5, 3.0, 0.0, 7.0], [2.0, 0.25, 1.0, 5.0]])
    st = orc.fp8.decode_state(cq[0, :2], fr)
    for s_ in range(2):
        for r in range(4):
            for d in range(5):
                assert st[s_, r, d] == FP8_ALL[int(cq[0, s_, r, d])] * fr[s_, r]


def _fp8_table():
    """Every finite E4M3 value by enumeration of (sign, exponent, mantissa) fields."""
    t = {}
    for c in range(256):
        sgn, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        t[c] = -mag if sgn else mag
    return t


FP8_ALL = _fp8_table()


PINS = [check_golden, check_bruteforce_loops, check_states_vs_sdpa, check_merge_equals_full,
        check_identity_bitexact, check_closed_forms, check_contribution, check_reuse,
        check_compose_groups, check_mse, check_planner_golden, check_norms, check_planner_invariants, check_epsilon, check_fp8]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


# --------------------------------------------------------------------------- #
# Invariants under random orders and bracketings (hypothesis)
# --------------------------------------------------------------------------- #

@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), k=st.integers(1, 9), n_empty=st.integers(0, 3))
def test_merge_any_order_any_bracketing(seed, k, n_empty):
    g = np.random.default_rng(seed)
    rows, D = 4, 6
    outs = g.standard_normal((k + n_empty, rows, D))
    lses = g.standard_normal((k + n_empty, rows)) * 5
    outs[k:] = 0
    lses[k:] = -np.inf
    ref_o, ref_l = oracle.merge(outs, lses)
    # random permutation, then a random binary tree of pairwise merges
    states = [(outs[i], lses[i]) for i in g.permutation(k + n_empty)]
    while len(states) > 1:
        j = int(g.integers(0, len(states) - 1))
        states[j:j + 2] = [oracle.merge_pair(states[j], states[j + 1])]
    np.testing.assert_allclose(states[0][0], ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(states[0][1], ref_l, rtol=0, atol=1e-12)


def test_tiny_fp32_workload_shuffled_merge_is_full_attention():
    """The tiny fp32 workload: per-partition states merged in the shuffled order equal full softmax attention."""
    w = inputs.tiny_fp32()
    o, l = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    order = w.merge_order
    assert sorted(order) == [0, 1, 2, 3] and order != [0, 1, 2, 3]
    m_o, m_l = oracle.merge(o[order], l[order])
    np.testing.assert_allclose(m_o, sdpa(w.q.double(), w.k.double(), w.v.double(), w.scale), rtol=0, atol=1e-12)
    np.testing.assert_allclose(m_l, torch_lse(w.q.double(), w.k.double(), w.scale), rtol=0, atol=1e-12)


@pytest.mark.slow
def test_smooth_component_gives_spatial_locality():
    """Long-video recipe (reduced: 8 frames, 2 heads, 8 partitions): mean weight falls with distance."""
    w = inputs.long_video(frames=8, H=2, P=8)
    _, l = oracle.partition_states(w.q[:, :, ::16], w.k, w.v, w.ranges, w.scale)
    wts, _ = oracle.contribution(l.reshape(w.P, -1), l.shape[-1])
    mean_w = wts.mean(1)
    by_dist = [np.mean([mean_w[i] for i in range(w.P) if abs(i - w.local) == d]) for d in range(4)]
    assert all(by_dist[d] > by_dist[d + 1] for d in range(3)), by_dist
    assert by_dist[0] > 10 * by_dist[3]


# --------------------------------------------------------------------------- #
# Planted mistakes: every plausible slip in the oracle must fail some pin
# --------------------------------------------------------------------------- #

MUTANTS = {
    "fp8 exponent bias off by one": ("BIAS = 7", "BIAS = 8", "fp8.py"),
    "fp8 subnormal exponent": ("np.exp2(1.0 - BIAS)", "np.exp2(-BIAS)", "fp8.py"),
    "fp8 mantissa width": ("(1.0 + m / 8.0)", "(1.0 + m / 16.0)", "fp8.py"),
    "fp8 sign bit": ("np.where(c & 0x80, -1.0, 1.0)", "np.where(c & 0x40, -1.0, 1.0)", "fp8.py"),
    "fp8 scale of the wrong head": ("vals * s[:, :, None, None]", "vals * s[:, ::-1, None, None]", "fp8.py"),
    "fp8 state factor of the wrong row": ("dtype=np.float64)[..., None]", "dtype=np.float64)[..., ::-1, None]",
                                          "fp8.py"),
    # states.py
    "scale dropped": ("z = scale * (q @ k.T)", "z = (q @ k.T)"),
    "keys used as values": ("return p @ v, lse", "return p @ k, lse"),
    "head index mixed up": ("k[b, h, s:e], v[b, h, s:e]", "k[b, -1 - h, s:e], v[b, -1 - h, s:e]"),
    "max left out of LSE": ("lse = m + np.log(", "lse = np.log("),
    "OUT not normalised": ("p = np.exp(z - lse[:, None])", "p = np.exp(z - m[:, None])"),
    "merge weights not normalised": ("weights = a / S1[None]", "weights = a"),
    "merge LSE without log": ("M0 + np.log(S1)", "M0 + S1"),
    "merge sign flipped": ("a = np.exp(lses - M0[None])", "a = np.exp(M0[None] - lses)"),
    "empty LSE zero": ("np.full(sq, NEG_INF)", "np.zeros(sq)"),
    "contribution not normalised": ("np.exp(lse - np.where(empty, 0.0, lstar)[None])", "np.exp(lse)"),
    "score sums instead of means": (".mean(axis=2).T", ".sum(axis=2).T"),
    "reuse caches the new step": ("c_out, c_lse = merge(out_t[far], lse_t[far])",
                                  "c_out, c_lse = merge(_f64(out_t1)[far], _f64(lse_t1)[far])"),
    "mse as a root": ("return float(np.mean((_f64(a) - _f64(b)) ** 2))",
                      "return float(np.sqrt(np.mean((_f64(a) - _f64(b)) ** 2)))"),
    "mse of absolute differences": ("np.mean((_f64(a) - _f64(b)) ** 2)", "np.mean(np.abs(_f64(a) - _f64(b)))"),
    "mse summed": ("np.mean((_f64(a) - _f64(b)) ** 2)", "np.sum((_f64(a) - _f64(b)) ** 2)"),
    "range end off by one": ("k[b, h, s:e], v[b, h, s:e]", "k[b, h, s:e + 1], v[b, h, s:e + 1]"),
    "group overlaps the next one": ("merge(outs[k:k + group], lses[k:k + group])",
                                    "merge(outs[k:k + group + 1], lses[k:k + group + 1])"),
    "groups skip a partition": ("for k in range(0, P, group)]", "for k in range(0, P, group + 1)]"),
    # planner.py
    "alpha inverted": ("return n / n[local]", "return n[local] / n", "planner.py"),
    "drift not scaled by alpha": ("return _f64(alpha) * float(local_drift)",
                                  "return np.ones_like(_f64(alpha)) * float(local_drift)", "planner.py"),
    "group boundary off by one": ("range(k, min(k + group, P))", "range(k, min(k + group + 1, P))", "planner.py"),
    "weights left out of ASE": ("sum(w[j] * d[j] for j in g)", "sum(d[j] for j in g)", "planner.py"),
    "local group not forced": ("compute[local // group] = 1", "pass", "planner.py"),
    "reuse above the threshold": ("compute = (ase > eps)", "compute = (ase < eps)", "planner.py"),
    "percentile off by one": ("np.sort(others)[m - 1]", "np.sort(others)[min(m, len(others) - 1)]", "planner.py"),
    "local group kept in percentile": ("if k != local // group]", "if True]", "planner.py"),
    "norm left squared": ("return np.sqrt(np.einsum(\"ij,ij->i\", d, d))", "return np.einsum(\"ij,ij->i\", d, d)",
                          "planner.py"),
    "difference taken as a sum": ("d = a if b is None else a - _f64(b)", "d = a if b is None else a + _f64(b)",
                                  "planner.py"),
    "anchor on small drift": ("return float(local_drift) > float(eps_local)",
                              "return float(local_drift) < float(eps_local)", "planner.py"),
}


def mutant_module(old, new, file="states.py"):
    """A stand-in for the oracle package with `old` replaced by `new` in one of its sources."""
    src_path = os.path.join(os.path.dirname(oracle.__file__), file)
    src = open(src_path).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant_" + file[:-3])
    mod.__file__ = src_path
    exec(compile(src.replace(old, new), src_path, "exec"), mod.__dict__)
    if file in ("planner.py", "fp8.py"):
        pkg = types.SimpleNamespace(**{k: getattr(oracle, k) for k in dir(oracle) if not k.startswith("_")})
        setattr(pkg, file[:-3], mod)
        return pkg
    mod.planner = oracle.planner
    mod.fp8 = oracle.fp8
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    mod = mutant_module(*MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"
