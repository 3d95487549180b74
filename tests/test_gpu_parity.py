"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (max-abs): bf16 inputs 2e-2 on OUT and 1e-3 on LSE; fp32 inputs 1e-5 on
both; partition weights 1e-5 (fp32 arithmetic on the same LSE); empty states
must be exactly (0, -inf). Small cases span several tiles with ragged tails and
are checked element by element; so are the image and video DiT workloads at full
size, and every row of three heads of the long-video and selective-reuse workloads.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from sequence_dit_amd import _native as N
from sequence_dit_amd import inputs
from sequence_dit_amd.reuse import SelectiveReuse

pytestmark = pytest.mark.gpu

BF16_OUT, BF16_LSE, F32_TOL = 2e-2, 1e-3, 1e-5
DEV = "cuda:0"


def note(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(N.LIB_PATH):
        pytest.fail("libas_attn.so is not built")
    N.lib()


def to_dev(t):
    return t.to(DEV)


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


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_small_ragged(D):
    """Two query tiles with a ragged tail; ranges: ragged, single key, empty, tile-aligned, overlapping, full."""
    w = inputs.small_case(7 + D, 2, 3, 300, 1000, D, RAGGED)
    note(f"bf16 small ragged D={D} B=2 H=3 Sq=300 Skv=1000 P={len(RAGGED)}")
    out, lse = N.partition_attn(to_dev(w.q), to_dev(w.k), to_dev(w.v), w.ranges, w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"bf16 D={D}")


SPLIT_RANGES = [(0, 400), (400, 400), (400, 401), (401, 1200), (1200, 1333), (1333, 2100), (2100, 3000), (0, 3000)]


@pytest.mark.parametrize("D", [128, 64])
def test_partial_tiles_issued_on_their_own_compute_units(D):
    """22 heads x 8 partitions x 520 query rows: two full query tiles and an 8-row one per
    unit, a shape whose launch keeps part of each XCD's compute units on the partial tiles
    (the issue order changes; every tile must still be computed once). Every element against
    the oracle; ragged, empty, single-key and overlapping ranges."""
    w = inputs.small_case(61 + D, 1, 22, 520, 3000, D, SPLIT_RANGES)
    note(f"partial-tile issue order D={D} B=1 H=22 Sq=520 Skv=3000 P={len(SPLIT_RANGES)}")
    out, lse = N.partition_attn(to_dev(w.q), to_dev(w.k), to_dev(w.v), w.ranges, w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"issue order D={D}")


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_max_partitions(D):
    """The largest number of partitions one launch takes (AS_MAX_PARTITIONS = 256; the ranges
    travel in the kernel's arguments): empty, single-key and overlapping ranges among them,
    a 40-row query shard (one partial query tile). Every element against the oracle."""
    ranges = inputs.random_ranges(D, 1500, N.AS_MAX_PARTITIONS)
    w = inputs.small_case(71 + D, 1, 2, 40, 1500, D, ranges)
    note(f"bf16 max partitions D={D} B=1 H=2 Sq=40 Skv=1500 P={len(ranges)}")
    out, lse = N.partition_attn(to_dev(w.q), to_dev(w.k), to_dev(w.v), w.ranges, w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"max partitions D={D}")


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_strided_inputs_and_guarded_outputs(D):
    """Non-contiguous q/k/v views and outputs followed by canaries that must stay untouched."""
    B, H, Sq, Skv = 1, 2, 130, 333
    w = inputs.small_case(21, B, H, Sq, Skv, D, [(0, 333), (5, 70), (300, 333)])
    qbig = torch.zeros(B, H, Sq + 16, D + 64, dtype=torch.bfloat16)
    qbig[:, :, 8:8 + Sq, :D] = w.q
    kbig = torch.zeros(B, H + 1, Skv, D + 8, dtype=torch.bfloat16)
    vbig = torch.zeros(B, H + 1, Skv, D + 8, dtype=torch.bfloat16)
    kbig[:, 1:, :, :D] = w.k
    vbig[:, 1:, :, :D] = w.v
    qd, kd, vd = to_dev(qbig)[:, :, 8:8 + Sq, :D], to_dev(kbig)[:, 1:, :, :D], to_dev(vbig)[:, 1:, :, :D]
    P = len(w.ranges)
    n_out, n_lse = P * B * H * Sq * D, P * B * H * Sq
    guard = 4096
    obuf = torch.full((n_out + guard,), 12345.0, device=DEV)
    lbuf = torch.full((n_lse + guard,), 12345.0, device=DEV)
    note(f"bf16 strided views + guarded outputs D={D}")
    out, lse = N.partition_attn(qd, kd, vd, w.ranges, w.scale, out=obuf[:n_out].view(P, B, H, Sq, D),
                                lse=lbuf[:n_lse].view(P, B, H, Sq))
    torch.cuda.synchronize()
    assert torch.all(obuf[n_out:] == 12345.0) and torch.all(lbuf[n_lse:] == 12345.0), "write past the end"
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, "bf16 strided")


# The fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) does not round its 64-product sums like
# fp32 round-to-nearest: products are aligned to the largest one and the rest keep about 17
# to 18 bits below its leading bit (an in-bounds check of the instruction on chosen codes:
# addends 2^-15 of the largest lose up to ~0.55 of their value each; equal-magnitude products
# sum exactly; on full-range random codes a 64-product block is off by up to 64 * 2^-17 of its
# largest product). The model used for fp8 scores: each 64-product block is off by at most
# 64 * 2^-16 * (its largest |q_d k_d|), the blocks then add in fp32.
# test_fp8_single_key_scores_within_truncation_model pins this model through the C ABI.
FP8_BLOCK, FP8_ALIGN_BITS = 64, 16


def fp8_score_bound(qd, kd, ranges, scale):
    """Per-element bound [P, B, H, Sq] on |LSE - LSE_exact| for fp8 q/k (decoded values qd, kd):
    the truncation model above for each score, the largest over the range (LSE is a smooth
    maximum), |scale| times, plus the 1e-3 LSE tolerance of bf16 inputs."""
    qa = np.abs(np.asarray(qd, dtype=np.float64))
    ka = np.abs(np.asarray(kd, dtype=np.float64))
    D = qa.shape[-1]
    err = np.zeros(qa.shape[:-1] + (ka.shape[-2],))
    for c in range(0, D, FP8_BLOCK):
        prod = qa[..., :, None, c:c + FP8_BLOCK] * ka[..., None, :, c:c + FP8_BLOCK]   # [B,H,Sq,Skv,64]
        err += FP8_BLOCK * 2.0 ** -FP8_ALIGN_BITS * prod.max(axis=-1) + 2.0 ** -23 * prod.sum(axis=-1)
    bounds = []
    for s, e in ranges:
        worst = err[..., s:e].max(axis=-1) if e > s else np.zeros(err.shape[:-1])
        bounds.append(BF16_LSE + abs(scale) * worst)
    return np.stack(bounds)


def score_rounding_bound(q, k, ranges, scale, unit=2.0 ** -24):
    """Per-element bound [P, B, H, Sq] on |LSE - LSE_exact| for scores accumulated in fp32.

    The products q_d * k_d of bf16 values are exact in fp32; a D-term sum accumulated in fp32
    is off by at most D * 2^-24 * sum_d |q_d k_d| (the gamma_D bound of floating-point
    summation, to first order), so each scaled score by that times |scale|. LSE is a smooth
    maximum of the scores, so it moves by at most the largest score error over the range. The
    1e-3 LSE tolerance of bf16 inputs is added for the softmax, exponential and log."""
    qa = np.abs(np.asarray(q, dtype=np.float64))
    ka = np.abs(np.asarray(k, dtype=np.float64))
    D = qa.shape[-1]
    absdot = qa @ np.swapaxes(ka, -1, -2)            # [B, H, Sq, Skv]
    bounds = []
    for s, e in ranges:
        worst = absdot[..., s:e].max(axis=-1) if e > s else np.zeros(absdot.shape[:-1])
        bounds.append(BF16_LSE + abs(scale) * D * unit * worst)
    return np.stack(bounds)


def check_lse_within(lse, l_ref, bound, what):
    got = lse.detach().cpu().double().numpy()
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(got), ~fin), f"{what}: -inf pattern differs"
    err = np.abs(got[fin] - l_ref[fin])
    note(f"{what}: LSE max-abs error {err.max():.3e}, bound {bound[fin].min():.3e}..{bound[fin].max():.3e}, "
         f"worst error/bound {np.max(err / bound[fin]):.3f}")
    assert np.all(err <= bound[fin]), f"{what}: LSE error {err.max():.3e} above the accumulation bound"


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_large_logits_stay_finite(D):
    """Scores scaled x100 (very peaked softmax, many lazy rescales, |LSE| up to ~300): no overflow,
    NaN, or loss of parity; the 17-key partition exercises the tail mask at both tile sizes. LSE is
    held to the 1e-3 LSE tolerance of bf16 inputs (a rescale slip that lost a percent of a partition's mass would
    move it by 1e-2); the fp32 score-accumulation bound of these inputs (score_rounding_bound, a few
    1e-3) is larger, and the errors measured on the GPU are below 1e-4."""
    w = inputs.small_case(31 if D == 128 else 95, 1, 2, 64, 500, D, [(0, 500), (0, 17), (250, 500)])
    note(f"bf16 large logits D={D}")
    out, lse = N.partition_attn(to_dev(w.q), to_dev(w.k), to_dev(w.v), w.ranges, 100 * w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, 100 * w.scale)
    check_lse_within(lse, l_ref, np.full(l_ref.shape, BF16_LSE), f"bf16 x100 logits D={D}")
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"bf16 x100 logits D={D}")


ZERO_SCALE_RANGES = [(0, 17), (17, 300), (5, 5), (299, 300), (3, 260)]


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_zero_scale_weighs_keys_equally(D):
    """scale = 0: every key of a range weighs e^0, so OUT = mean of V over the range and LSE = ln n
    (the 17-key and 257-key ranges end inside a key tile: the tail mask must not turn 0 * -inf into NaN)."""
    w = inputs.small_case(60 + D, 1, 2, 40, 300, D, ZERO_SCALE_RANGES)
    note(f"bf16 zero scale D={D}")
    out, lse = N.partition_attn(to_dev(w.q), to_dev(w.k), to_dev(w.v), w.ranges, 0.0)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, 0.0)
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"bf16 zero scale D={D}")
    v = w.v.double().numpy()
    for i, (s, e) in enumerate(w.ranges):
        if e > s:
            np.testing.assert_allclose(lse[i].cpu().double().numpy(), math.log(e - s), rtol=0, atol=1e-6)
            mean_v = v[:, :, s:e].mean(axis=2)[:, :, None, :]
            assert np.abs(out[i].cpu().double().numpy() - mean_v).max() <= 1e-5


@pytest.mark.parametrize("D", [128, 64])
def test_fp8_zero_and_negative_factors(D):
    """fp8 factors are device data of any sign: a zero factor weighs the keys equally, a negative
    product of factors negates the scores (both against the oracle on the decoded values)."""
    w = inputs.small_case_fp8(70 + D, 1, 3, 40, 300, D, ZERO_SCALE_RANGES)
    q_scale = w.q_scale.clone()
    k_scale = w.k_scale.clone()
    q_scale[0, 0] = 0.0        # head 0: zero factor
    k_scale[0, 1] *= -1.0      # head 1: negative product
    q_scale[0, 2] *= -1.0      # head 2: two negative factors, positive product
    k_scale[0, 2] *= -1.0
    note(f"fp8 zero and negative factors D={D}")
    out, lse = N.partition_attn_fp8(to_dev(w.q8), to_dev(w.k8), to_dev(w.v), to_dev(q_scale), to_dev(k_scale),
                                    w.ranges, w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = fp8_reference(w, w.q8, w.k8, q_scale, k_scale, w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"fp8 factors of any sign D={D}")


def fp8_reference(w, q8, k8, q_scale, k_scale, ranges, scale):
    """Oracle states on the values the fp8 codes stand for (decoded by the oracle)."""
    qd = oracle.fp8.dequantize(q8.cpu().view(torch.uint8).numpy(), q_scale.cpu().numpy())
    kd = oracle.fp8.dequantize(k8.cpu().view(torch.uint8).numpy(), k_scale.cpu().numpy())
    return oracle.partition_states(qd, kd, w.v if w is not None else None, ranges, scale)


@pytest.mark.parametrize("state", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [128, 64])
def test_fp8_small_ragged(D, state):
    """fp8 E4M3 q/k with per-(b, h) factors, bf16 v: ragged, single-key, empty, overlapping and full ranges."""
    w = inputs.small_case_fp8(50 + D, 2, 3, 300, 1000, D, RAGGED)
    note(f"fp8 small ragged D={D} state={state} B=2 H=3 Sq=300 Skv=1000 P={len(RAGGED)}")
    out, lse = N.partition_attn_fp8(to_dev(w.q8), to_dev(w.k8), to_dev(w.v), to_dev(w.q_scale),
                                    to_dev(w.k_scale), w.ranges, w.scale, state_dtype=state)
    torch.cuda.synchronize()
    o_ref, l_ref = fp8_reference(w, w.q8, w.k8, w.q_scale, w.k_scale, w.ranges, w.scale)
    check_states(out.float(), lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"fp8 D={D} {state}")


def test_selective_reuse_with_fp8_inputs():
    """The reuse step on fp8 q/k: anchor states at t, 2 fresh partitions at t+1 composed with the
    cached composition of the other 6, against the oracle's reuse step on the decoded states."""
    ranges = inputs.equal_ranges(1024, 8)
    w = inputs.small_case_fp8(90, 1, 2, 300, 1024, 128, ranges)
    w1 = inputs.small_case_fp8(91, 1, 2, 300, 1024, 128, ranges)
    near = [3, 4]
    runner = SelectiveReuse(1, 2, 300, 128, ranges, near, DEV, w.scale)
    note("selective reuse with fp8 q/k, P=8, 2 fresh")
    runner.anchor(to_dev(w.q8), to_dev(w.k8), to_dev(w.v), (to_dev(w.q_scale), to_dev(w.k_scale)))
    out, lse = runner.step(to_dev(w1.q8), to_dev(w1.k8), to_dev(w1.v), (to_dev(w1.q_scale), to_dev(w1.k_scale)))
    torch.cuda.synchronize()
    o_t, l_t = fp8_reference(w, w.q8, w.k8, w.q_scale, w.k_scale, ranges, w.scale)
    o_t1, l_t1 = fp8_reference(w1, w1.q8, w1.k8, w1.q_scale, w1.k_scale, ranges, w.scale)
    ref_out, ref_lse, c_out, c_lse = oracle.selective_reuse(o_t, l_t, o_t1, l_t1, near)
    check_states(runner.cached_out, runner.cached_lse, c_out, c_lse, BF16_OUT, BF16_LSE, "fp8 cached state")
    check_states(out, lse, ref_out, ref_lse, BF16_OUT, BF16_LSE, "fp8 reuse result")
    with pytest.raises(ValueError):
        runner.step(to_dev(w1.q8), to_dev(w1.k8), to_dev(w1.v))


def test_fp8_path_equals_bf16_path_on_the_same_values():
    """Codes of moderate size with factors 1 are exact in bf16, so both paths score the same Q and K.
    The fp8 MFMA sums 64 products per instruction and rounds differently from four bf16 MFMAs (LSE
    differences up to ~2e-4 were seen on LSE values of 8-16), and P's bf16 rounding can flip with it;
    both stay inside the oracle tolerances. A K/Q byte-order slip in the fp8 operands would give O(1)
    differences."""
    w = inputs.small_case(77, 1, 2, 257, 700, 128, [(0, 700), (3, 300), (650, 700)])
    q8 = (2 * w.q.float()).to(torch.float8_e4m3fn)
    k8 = (2 * w.k.float()).to(torch.float8_e4m3fn)
    ones = torch.ones(1, 2, device=DEV)
    note("fp8 path vs bf16 path on identical values")
    o8, l8 = N.partition_attn_fp8(to_dev(q8), to_dev(k8), to_dev(w.v), ones, ones, w.ranges, w.scale)
    o16, l16 = N.partition_attn(to_dev(q8.to(torch.bfloat16)), to_dev(k8.to(torch.bfloat16)), to_dev(w.v),
                                w.ranges, w.scale)
    torch.cuda.synchronize()
    assert (l8 - l16).abs().max().item() <= BF16_LSE
    assert (o8 - o16).abs().max().item() <= 1e-2


@pytest.mark.parametrize("D", [128, 64])
def test_fp8_single_key_scores_within_truncation_model(D):
    """Single-key ranges isolate one score: LSE = scale * <q, k> exactly and OUT = v, so the LSE
    error is the fp8 MFMA's error on that dot product (plus a few fp32 roundings). Codes span the
    whole E4M3 range (worst case for the aligned sums); every error must lie within the model of
    fp8_score_bound, and the errors must show that the instruction is not exact (else the model
    would be vacuous)."""
    g = np.random.default_rng(300 + D)
    B, H, Sq, Skv = 1, 2, 64, 200
    codes = lambda n: g.integers(0, 256, size=n).astype(np.uint8)
    q8 = codes((B, H, Sq, D))
    k8 = codes((B, H, Skv, D))
    q8[(q8 & 0x7F) == 0x7F] = 0x38    # no NaN codes
    k8[(k8 & 0x7F) == 0x7F] = 0x38
    ranges = [(j, j + 1) for j in range(0, Skv, 2)]
    ones = torch.ones(B, H)
    v = torch.from_numpy(g.standard_normal((B, H, Skv, D)).astype(np.float32)).to(torch.bfloat16)
    scale = 2.0 ** -12   # keeps the scores of full-range codes (|dot| up to ~1e7) moderate
    note(f"fp8 single-key scores D={D}")
    qt = torch.from_numpy(q8).view(torch.float8_e4m3fn)
    kt = torch.from_numpy(k8).view(torch.float8_e4m3fn)
    out, lse = N.partition_attn_fp8(to_dev(qt), to_dev(kt), to_dev(v), to_dev(ones), to_dev(ones), ranges, scale)
    torch.cuda.synchronize()
    qd = oracle.fp8.dequantize(q8, ones.numpy())
    kd = oracle.fp8.dequantize(k8, ones.numpy())
    o_ref, l_ref = oracle.partition_states(qd, kd, v, ranges, scale)
    got = lse.cpu().double().numpy()
    bound = fp8_score_bound(qd, kd, ranges, scale) - BF16_LSE + 8 * 2.0 ** -24 * np.abs(l_ref)
    err = np.abs(got - l_ref)
    note(f"fp8 single-key D={D}: |score error| max {err.max():.3e}, worst error/model {np.max(err / bound):.3f}")
    assert np.all(err <= bound)
    assert err.max() > 8 * 2.0 ** -24 * np.abs(l_ref).max(), "the fp8 sums were exact: model untested"
    assert np.abs(out.float().cpu().numpy() - np.asarray(o_ref)).max() == 0   # OUT = v exactly


@pytest.mark.parametrize("D", [128, 64])
def test_fp8_large_logits_stay_finite(D):
    """fp8 q/k with the softmax scale x100 (very peaked, several lazy rescales): finite and at parity,
    LSE within the fp8 MFMA's truncation model (fp8_score_bound) of the decoded values. The
    softmax itself is the bf16 path's and is held to 1e-3 at x100 there."""
    w = inputs.small_case_fp8(33 + D, 1, 2, 64, 500, D, [(0, 500), (0, 17), (250, 500)])
    note(f"fp8 large logits D={D}")
    out, lse = N.partition_attn_fp8(to_dev(w.q8), to_dev(w.k8), to_dev(w.v), to_dev(w.q_scale), to_dev(w.k_scale),
                                    w.ranges, 100 * w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = fp8_reference(w, w.q8, w.k8, w.q_scale, w.k_scale, w.ranges, 100 * w.scale)
    qd = oracle.fp8.dequantize(w.q8.view(torch.uint8).numpy(), w.q_scale.numpy())
    kd = oracle.fp8.dequantize(w.k8.view(torch.uint8).numpy(), w.k_scale.numpy())
    bound = fp8_score_bound(qd, kd, w.ranges, 100 * w.scale)
    check_lse_within(lse, l_ref, bound, f"fp8 x100 logits D={D}")
    check_states(out, lse, o_ref, l_ref, BF16_OUT, bound.max(), f"fp8 x100 logits D={D}")


def test_fp8_strided_inputs_and_guarded_outputs():
    """fp8 views with padded rows and an extra head; outputs followed by canaries."""
    D, B, H, Sq, Skv = 128, 1, 2, 130, 333
    w = inputs.small_case_fp8(22, B, H, Sq, Skv, D, [(0, 333), (5, 70), (300, 333)])
    qbig = torch.zeros(B, H, Sq + 16, D + 16, dtype=torch.uint8)
    qbig[:, :, 8:8 + Sq, :D] = w.q8.view(torch.uint8)
    kbig = torch.zeros(B, H + 1, Skv, D + 16, dtype=torch.uint8)
    vbig = torch.zeros(B, H + 1, Skv, D + 16, dtype=torch.bfloat16)
    kbig[:, 1:, :, :D] = w.k8.view(torch.uint8)
    vbig[:, 1:, :, :D] = w.v
    fp8 = torch.float8_e4m3fn
    qd = to_dev(qbig).view(fp8)[:, :, 8:8 + Sq, :D]
    kd = to_dev(kbig).view(fp8)[:, 1:, :, :D]
    vd = to_dev(vbig)[:, 1:, :, :D]
    P = len(w.ranges)
    n_out, n_lse = P * B * H * Sq * D, P * B * H * Sq
    guard = 4096
    obuf = torch.full((n_out + guard,), 12345.0, device=DEV)
    lbuf = torch.full((n_lse + guard,), 12345.0, device=DEV)
    note("fp8 strided views + guarded outputs")
    out, lse = N.partition_attn_fp8(qd, kd, vd, to_dev(w.q_scale), to_dev(w.k_scale), w.ranges, w.scale,
                                    out=obuf[:n_out].view(P, B, H, Sq, D), lse=lbuf[:n_lse].view(P, B, H, Sq))
    torch.cuda.synchronize()
    assert torch.all(obuf[n_out:] == 12345.0) and torch.all(lbuf[n_lse:] == 12345.0), "write past the end"
    o_ref, l_ref = fp8_reference(w, w.q8, w.k8, w.q_scale, w.k_scale, w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, "fp8 strided")


def test_f32_tiny_workload_shuffled_merge_equals_full_attention():
    """The tiny fp32 workload: states, then a merge in shuffled order, equal full attention within 1e-5."""
    w = inputs.tiny_fp32()
    note("f32 tiny workload")
    out, lse = N.partition_attn(to_dev(w.q), to_dev(w.k), to_dev(w.v), w.ranges, w.scale)
    order = w.merge_order
    m_out, m_lse = N.merge([out[i] for i in order], [lse[i] for i in order])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, F32_TOL, F32_TOL, "f32 states")
    f_out, f_lse = oracle.full_attention(w.q, w.k, w.v, w.scale)
    check_states(m_out, m_lse, f_out, f_lse, F32_TOL, F32_TOL, "f32 merged vs full attention")


@pytest.mark.parametrize("D", [128, 40, 8])
def test_f32_ragged(D):
    w = inputs.small_case(41 + D, 1, 2, 100, 300, D, [(0, 300), (3, 4), (4, 4), (37, 251)], dtype=torch.float32)
    note(f"f32 ragged D={D}")
    out, lse = N.partition_attn(to_dev(w.q), to_dev(w.k), to_dev(w.v), w.ranges, w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    check_states(out, lse, o_ref, l_ref, F32_TOL, F32_TOL, f"f32 D={D}")


# --------------------------------------------------------------------------- #
# merge
# --------------------------------------------------------------------------- #

def random_states(seed, n, rows, D, n_empty=0):
    g = np.random.default_rng(seed)
    outs = g.standard_normal((n, rows, D)).astype(np.float32)
    lses = (g.standard_normal((n, rows)) * 4).astype(np.float32)
    if n_empty:
        idx = g.choice(n * rows, size=n_empty, replace=False)
        outs.reshape(n * rows, D)[idx] = 0
        lses.reshape(-1)[idx] = -np.inf
    return outs, lses


@pytest.mark.parametrize("n,rows,D", [(2, 1000, 128), (5, 777, 128), (32, 300, 128), (28, 129, 64), (64, 33, 4),
                                      (3, 50, 1024), (9, 301, 32), (64, 77, 256), (17, 90, 40), (1, 20, 128)])
def test_merge_matches_oracle(n, rows, D):
    outs, lses = random_states(n * 1000 + D, n, rows, D, n_empty=rows // 3)
    # one row where every input is empty
    outs[:, 0] = 0
    lses[:, 0] = -np.inf
    note(f"merge n={n} rows={rows} D={D}")
    od, ld = to_dev(torch.from_numpy(outs)), to_dev(torch.from_numpy(lses))
    m_out, m_lse = N.merge(list(od), list(ld))
    torch.cuda.synchronize()
    r_out, r_lse = oracle.merge(outs, lses)
    check_states(m_out, m_lse, r_out, r_lse, F32_TOL, F32_TOL, f"merge n={n}")


def test_merge_with_empty_state_is_bitwise_identity():
    outs, lses = random_states(5, 1, 513, 128)
    outs[0, 3, 5] = -0.0
    note("merge identity")
    x_out, x_lse = to_dev(torch.from_numpy(outs[0])), to_dev(torch.from_numpy(lses[0]))
    e_out, e_lse = torch.zeros_like(x_out), torch.full_like(x_lse, float("-inf"))
    for ins in ([x_out, e_out], [e_out, x_out], [e_out, x_out, e_out]):
        lins = [x_lse if t is x_out else e_lse for t in ins]
        m_out, m_lse = N.merge(ins, lins)
        torch.cuda.synchronize()
        assert torch.equal(m_out.view(torch.int32), x_out.view(torch.int32)), "OUT bits changed"
        assert torch.equal(m_lse.view(torch.int32), x_lse.view(torch.int32)), "LSE bits changed"
    m_out, m_lse = N.merge([e_out, e_out], [e_lse, e_lse])
    torch.cuda.synchronize()
    assert torch.all(m_out == 0) and torch.all(torch.isneginf(m_lse))


# --------------------------------------------------------------------------- #
# Compact (bf16 OUT) states and group-wise composition
# --------------------------------------------------------------------------- #

def bf16_close(got, ref, what):
    """Within one bf16 rounding of the reference (2^-8 relative) plus fp32 noise."""
    err = np.abs(got - ref) - (np.abs(ref) * 2.0 ** -8 + 1e-6)
    assert np.all(err <= 0), f"{what}: off by more than a bf16 rounding (worst excess {err.max():.3e})"


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_states_are_rounded_fp32_states(D):
    w = inputs.small_case(11 + D, 1, 3, 300, 1000, D, RAGGED)
    note(f"bf16 states D={D}")
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    o32, l32 = N.partition_attn(q, k, v, w.ranges, w.scale)
    o16, l16 = N.partition_attn_states(q, k, v, w.ranges, w.scale, torch.bfloat16)
    torch.cuda.synchronize()
    # the same arithmetic, then one round-to-nearest-even of OUT
    assert o16.dtype == torch.bfloat16 and torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(l16, l32)
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    check_states(o16.float(), l16, o_ref, l_ref, BF16_OUT, BF16_LSE, f"bf16 states D={D}")


def test_f32_inputs_with_bf16_states():
    w = inputs.small_case(12, 1, 2, 70, 300, 40, [(0, 100), (100, 300), (50, 51), (7, 7)], dtype=torch.float32)
    note("f32 inputs, bf16 states")
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    o32, l32 = N.partition_attn(q, k, v, w.ranges, w.scale)
    o16, l16 = N.partition_attn_states(q, k, v, w.ranges, w.scale, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(l16, l32)
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    fin = np.isfinite(l_ref)
    bf16_close(o16.float().cpu().double().numpy()[fin], o_ref[fin], "f32 inputs, bf16 OUT")
    assert np.abs(l16.cpu().double().numpy()[fin] - l_ref[fin]).max() <= F32_TOL


@pytest.mark.parametrize("n,rows,D,in_dt,out_dt", [
    (28, 300, 128, torch.bfloat16, torch.bfloat16), (5, 777, 128, torch.bfloat16, torch.float32),
    (4, 129, 64, torch.float32, torch.bfloat16), (64, 33, 4, torch.bfloat16, torch.bfloat16),
    (9, 301, 40, torch.bfloat16, torch.float32), (3, 50, 1024, torch.float32, torch.float32)])
def test_merge_states_matches_oracle(n, rows, D, in_dt, out_dt):
    outs, lses = random_states(n * 7 + D, n, rows, D, n_empty=rows // 3)
    outs[:, 0] = 0
    lses[:, 0] = -np.inf
    note(f"merge_states n={n} rows={rows} D={D} {in_dt}->{out_dt}")
    od = to_dev(torch.from_numpy(outs)).to(in_dt)
    ld = to_dev(torch.from_numpy(lses))
    m_out, m_lse = N.merge_states(list(od), list(ld), out_dt)
    torch.cuda.synchronize()
    # the oracle composes exactly the stored inputs
    r_out, r_lse = oracle.merge(od.float().cpu().numpy(), lses)
    got = m_out.float().cpu().double().numpy()
    if out_dt == torch.float32:
        check_states(m_out, m_lse, r_out, r_lse, F32_TOL, F32_TOL, "merge_states")
    else:
        bf16_close(got, r_out, "merge_states bf16 OUT")
        fin = np.isfinite(r_lse)
        assert np.abs(m_lse.cpu().double().numpy()[fin] - r_lse[fin]).max() <= F32_TOL
        assert np.all(np.isneginf(m_lse.cpu().numpy()[~fin])) and np.all(got[~fin] == 0)
    if in_dt == torch.float32 and out_dt == torch.float32:
        f_out, f_lse = N.merge(list(od), list(ld))
        assert torch.equal(f_out, m_out) and torch.equal(f_lse, m_lse)


def test_merge_states_bf16_identity():
    outs, lses = random_states(6, 1, 257, 128)
    x = to_dev(torch.from_numpy(outs[0])).to(torch.bfloat16)
    xl = to_dev(torch.from_numpy(lses[0]))
    e, el = torch.zeros_like(x), torch.full_like(xl, float("-inf"))
    m_out, m_lse = N.merge_states([e, x, e], [el, xl, el], torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(m_out.view(torch.int16), x.view(torch.int16)) and torch.equal(m_lse, xl)


@pytest.mark.parametrize("P,group,rows,D,in_dt,out_dt", [
    (32, 4, 300, 128, torch.bfloat16, torch.bfloat16), (7, 3, 129, 64, torch.float32, torch.float32),
    (32, 8, 3840, 128, torch.float32, torch.bfloat16), (5, 64, 33, 4, torch.bfloat16, torch.float32),
    (256, 16, 20, 128, torch.bfloat16, torch.bfloat16), (6, 1, 50, 32, torch.float32, torch.float32)])
def test_compose_groups_matches_oracle(P, group, rows, D, in_dt, out_dt):
    outs, lses = random_states(P * 3 + group, P, rows, D, n_empty=rows // 2)
    outs[:, 1] = 0
    lses[:, 1] = -np.inf
    note(f"compose_groups P={P} group={group} rows={rows} D={D} {in_dt}->{out_dt}")
    od = to_dev(torch.from_numpy(outs)).to(in_dt)
    ld = to_dev(torch.from_numpy(lses))
    g_out, g_lse = N.compose_groups(od, ld, group, out_dt)
    torch.cuda.synchronize()
    r_out, r_lse = oracle.compose_groups(od.float().cpu().numpy(), lses, group)
    assert g_out.shape[0] == (P + group - 1) // group
    if out_dt == torch.float32:
        check_states(g_out, g_lse, r_out, r_lse, F32_TOL, F32_TOL, "compose_groups")
    else:
        bf16_close(g_out.float().cpu().double().numpy(), r_out, "compose_groups bf16 OUT")
        fin = np.isfinite(r_lse)
        assert np.abs(g_lse.cpu().double().numpy()[fin] - r_lse[fin]).max() <= F32_TOL
    # one launch over all groups gives, bit for bit, the per-group merges
    for k in range(0, P, max(1, P // 4 // group) * group):
        m_out, m_lse = N.merge_states(list(od[k:k + group]), list(ld[k:k + group]), out_dt)
        torch.cuda.synchronize()
        assert torch.equal(m_out, g_out[k // group]) and torch.equal(m_lse, g_lse[k // group]), k


def test_merge_tree_equals_flat_on_gpu():
    """Associativity and commutativity on the device: ((a,b),(c,(d,e))) equals the flat 5-way merge."""
    outs, lses = random_states(77, 5, 400, 128)
    od, ld = list(to_dev(torch.from_numpy(outs))), list(to_dev(torch.from_numpy(lses)))
    note("merge tree")
    ab = N.merge([od[1], od[0]], [ld[1], ld[0]])
    de = N.merge([od[4], od[3]], [ld[4], ld[3]])
    cde = N.merge([de[0], od[2]], [de[1], ld[2]])
    t_out, t_lse = N.merge([cde[0], ab[0]], [cde[1], ab[1]])
    f_out, f_lse = N.merge(od, ld)
    torch.cuda.synchronize()
    assert (t_out - f_out).abs().max().item() <= F32_TOL
    assert (t_lse - f_lse).abs().max().item() <= F32_TOL


# --------------------------------------------------------------------------- #
# contribution
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("P,rows,rpg", [(32, 2 * 3840, 3840), (5, 1000, 250), (8, 777, 777), (3, 64, 1), (256, 300, 100),
                                        (33, 500, 250), (100, 257, 257)])
def test_contribution_matches_oracle(P, rows, rpg):
    g = np.random.default_rng(P * 7 + rows)
    lse = (g.standard_normal((P, rows)) * 6).astype(np.float32)
    lse[0, :5] = -np.inf
    lse[:, 7] = -np.inf  # a row with every partition empty
    note(f"contribution P={P} rows={rows} rpg={rpg}")
    ld = to_dev(torch.from_numpy(lse))
    w, s = N.partition_contribution(ld, rpg)
    w2, s2 = N.partition_contribution(ld, rpg)
    torch.cuda.synchronize()
    w_ref, s_ref = oracle.contribution(lse, rpg)
    assert np.abs(w.cpu().double().numpy() - w_ref).max() <= F32_TOL
    assert np.abs(s.cpu().double().numpy() - s_ref).max() <= F32_TOL
    assert torch.equal(s, s2) and torch.equal(w, w2), "not deterministic"


# --------------------------------------------------------------------------- #
# Planner statistics
# --------------------------------------------------------------------------- #

NORM_RTOL = 1e-6   # fp64 sums rounded once to fp32 (unit roundoff 2^-24)
PLAN_RTOL = 1e-5   # fp32 arithmetic on a few terms per output


def test_contribution_large_lse_values():
    """LSE values near 1000 (scores of a x100 logit scale): the weights are softmaxes of LSE
    differences and must keep fp32 accuracy; forming L* = M + ln S first would round it to
    the ulp of M (6e-5 at 1000)."""
    g = np.random.default_rng(41)
    P, rows = 32, 1000
    lse = (1000.0 + 3.0 * g.standard_normal((P, rows))).astype(np.float32)
    lse[3, :50] = -np.inf
    note("contribution with LSE ~ 1000")
    w, sc = N.partition_contribution(torch.from_numpy(lse).to(DEV), 250)
    torch.cuda.synchronize()
    w_ref, s_ref = oracle.contribution(lse, 250)
    assert np.abs(w.cpu().double().numpy() - w_ref).max() <= F32_TOL
    assert np.abs(sc.cpu().double().numpy() - s_ref).max() <= F32_TOL


@pytest.mark.parametrize("diff", [False, True])
@pytest.mark.parametrize("P,n", [(1, 4), (3, 4100), (5, 0), (32, 300 * 128), (256, 64), (2, 3 * 262144 + 20),
                                 (1, 24 * 3840 * 128)])
def test_state_norms_matches_oracle(P, n, diff):
    g = np.random.default_rng(P * 13 + n + int(diff))
    a = g.standard_normal((P, n)).astype(np.float32)
    b = g.standard_normal((P, n)).astype(np.float32) if diff else None
    note(f"state norms P={P} n={n} diff={diff}")
    ad = to_dev(torch.from_numpy(a))
    bd = to_dev(torch.from_numpy(b)) if diff else None
    got = N.state_norms(ad, bd)
    again = N.state_norms(ad, bd)
    torch.cuda.synchronize()
    ref = oracle.planner.state_norm(a, b)
    np.testing.assert_allclose(got.cpu().double().numpy(), ref, rtol=NORM_RTOL, atol=0)
    assert torch.equal(got, again), "not deterministic"


def planner_inputs(P, seed):
    g = np.random.default_rng(seed)
    norms = g.uniform(0.1, 3.0, P).astype(np.float32)
    w = g.dirichlet(np.ones(P)).astype(np.float32)
    drift = np.float32(g.uniform(0.01, 0.5))
    return norms, w, drift


@pytest.mark.parametrize("P,local,group", [(32, 16, 4), (11, 4, 3), (8, 0, 8), (5, 4, 2), (256, 100, 16),
                                           (7, 3, 10), (1, 0, 1)])
def test_planner_decide_matches_oracle(P, local, group):
    norms, w, drift = planner_inputs(P, P + 1000 * local + group)
    note(f"planner decide P={P} local={local} group={group}")
    ase_ref = oracle.planner.planner(norms, drift, w, local, group, 0.0, 0.2)["ase"]
    for eps in (-np.inf, 0.0, float(np.median(ase_ref)), 1e9):
        eps32 = np.float32(eps)
        r = N.planner_decide(to_dev(torch.from_numpy(norms)), to_dev(torch.tensor([drift])),
                             to_dev(torch.from_numpy(w)), to_dev(torch.tensor([eps32])), local, group, 0.2)
        torch.cuda.synchronize()
        ref = oracle.planner.planner(norms, drift, w, local, group, float(eps32), 0.2)
        for key in ("alpha", "delta", "ase"):
            np.testing.assert_allclose(r[key].cpu().double().numpy(), ref[key], rtol=PLAN_RTOL, atol=0)
        # the decision is an integer taken on the GPU's own fp32 errors: the oracle takes it on the same numbers
        gpu_ase = r["ase"].cpu().double().numpy()
        assert np.array_equal(r["compute"].cpu().numpy(), oracle.planner.decide(gpu_ase, local, group, float(eps32)))
        assert int(r["anchor"].item()) == int(ref["anchor"])
    # the anchor flag on both sides of eps_local
    r = N.planner_decide(to_dev(torch.from_numpy(norms)), to_dev(torch.tensor([drift])), to_dev(torch.from_numpy(w)),
                         to_dev(torch.tensor([0.0])), local, group, float(drift) * 2)
    assert int(r["anchor"].item()) == 0


@pytest.mark.parametrize("P,local,group", [(32, 16, 4), (11, 4, 3), (256, 7, 2), (8, 0, 8), (5, 4, 1)])
def test_planner_epsilon_matches_oracle(P, local, group):
    g = np.random.default_rng(P * 31 + local + group)
    corr = g.uniform(0.0, 1.0, P).astype(np.float32)
    w = g.dirichlet(np.ones(P)).astype(np.float32)
    note(f"planner epsilon P={P} local={local} group={group}")
    for R in (0.0, 0.1, 1 / 3, 0.5, 0.75, 1.0):
        eps = N.planner_epsilon(to_dev(torch.from_numpy(corr)), to_dev(torch.from_numpy(w)), local, group, R)
        torch.cuda.synchronize()
        got = float(eps.item())
        ref = oracle.planner.epsilon(corr, w, local, group, R)
        if np.isinf(ref):
            assert got == -np.inf, (R, got)
        else:
            assert abs(got - ref) <= PLAN_RTOL * abs(ref), (R, got, ref)


# --------------------------------------------------------------------------- #
# Full-size workloads, sampled rows
# --------------------------------------------------------------------------- #

def sampled_reference(w, q, k, v, heads, rows_sel, ranges):
    qs = q[:, heads][:, :, rows_sel]
    return oracle.partition_states(qs, k[:, heads], v[:, heads], ranges, w.scale)


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_size_image_and_video(cfg):
    """The image and video DiT workloads at full size, every element of every partition state and
    of their composition (the launch configuration bench.py times)."""
    w = inputs.make(cfg)
    note(f"full size workload, all elements: {w.name}")
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    out, lse = N.partition_attn(q, k, v, w.ranges, w.scale)
    m_out, m_lse = N.merge(list(out), list(lse))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partition_states(w.q, w.k, w.v, w.ranges, w.scale)
    eo, el = check_states(out, lse, o_ref, l_ref, BF16_OUT, BF16_LSE, f"config {cfg} states")
    note(f"config {cfg}: OUT max-abs {eo:.3e}, LSE max-abs {el:.3e}")
    f_o, f_l = oracle.merge(o_ref, l_ref)
    check_states(m_out, m_lse, f_o, f_l, BF16_OUT, BF16_LSE, f"config {cfg} merged")


def fp8_full_size_check(w, q8, k8, qs, ks, heads, rs, what):
    """fp8 states of a full-size workload against the oracle on sampled rows of the decoded inputs."""
    out, lse = N.partition_attn_fp8(q8, k8, w.v_dev, qs, ks, w.ranges, w.scale)
    torch.cuda.synchronize()
    qsel = q8[:, heads][:, :, rs].cpu()
    ksel = k8[:, heads].cpu()
    qd = oracle.fp8.dequantize(qsel.view(torch.uint8).numpy(), qs[:, heads].cpu().numpy())
    kd = oracle.fp8.dequantize(ksel.view(torch.uint8).numpy(), ks[:, heads].cpu().numpy())
    o_ref, l_ref = oracle.partition_states(qd, kd, w.v[:, heads], w.ranges, w.scale)
    check_states(out[:, :, heads][:, :, :, rs], lse[:, :, heads][:, :, :, rs], o_ref, l_ref, BF16_OUT, BF16_LSE,
                 what)


def test_full_size_video_fp8():
    """Video DiT shape (D = 64, masked tiles) with fp8 q/k at full size, every element."""
    w = inputs.make(3)
    note(f"full size fp8 workload: {w.name}")
    q8, qs = inputs.quantize_fp8(to_dev(w.q))
    k8, ks = inputs.quantize_fp8(to_dev(w.k))
    w.v_dev = to_dev(w.v)
    fp8_full_size_check(w, q8, k8, qs, ks, list(range(w.H)), list(range(w.Sq)), "video fp8")


@pytest.fixture(scope="module")
def reuse_workload():
    return inputs.selective_reuse()


REUSE_HEADS = [0, 11, 23]


@pytest.fixture(scope="module")
def reuse_reference(reuse_workload):
    """Oracle states of every row of three heads at both steps of the selective-reuse workload."""
    w = reuse_workload
    rs = list(range(w.Sq))
    o_t, l_t = sampled_reference(w, w.q, w.k, w.v, REUSE_HEADS, rs, w.ranges)
    o_t1, l_t1 = sampled_reference(w, w.q1, w.k1, w.v1, REUSE_HEADS, rs, w.ranges)
    return o_t, l_t, o_t1, l_t1


def test_full_size_long_video_and_selective_reuse(reuse_workload, reuse_reference):
    """Long-video states (all 32 partitions) and the selective-reuse step at full size, every row of
    three heads."""
    w = reuse_workload
    note(f"full size workload: {w.name}")
    B, H, Sq, D = w.B, w.H, w.Sq, w.D
    runner = SelectiveReuse(B, H, Sq, D, w.ranges, w.near, DEV, w.scale)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    runner.anchor(q, k, v)
    del q, k, v
    q1, k1, v1 = to_dev(w.q1), to_dev(w.k1), to_dev(w.v1)
    r_out, r_lse = runner.step(q1, k1, v1)
    # full attention at t+1 on the GPU for the reported MSE
    full_out, full_lse = N.partition_attn(q1, k1, v1, w.ranges, w.scale)
    f_out, f_lse = N.merge(list(full_out), list(full_lse))
    torch.cuda.synchronize()

    heads = REUSE_HEADS
    rs = list(range(Sq))   # every row of three heads, all 32 partitions
    o_t, l_t, o_t1, l_t1 = reuse_reference
    check_states(runner.state_out[:, :, heads][:, :, :, rs], runner.state_lse[:, :, heads][:, :, :, rs],
                 o_t, l_t, BF16_OUT, BF16_LSE, "long video states (step t)")
    ref_out, ref_lse, c_out, c_lse = oracle.selective_reuse(o_t, l_t, o_t1, l_t1, w.near)
    check_states(runner.cached_out[:, heads][:, :, rs], runner.cached_lse[:, heads][:, :, rs], c_out, c_lse,
                 BF16_OUT, BF16_LSE, "cached composed state")
    check_states(r_out[:, heads][:, :, rs], r_lse[:, heads][:, :, rs], ref_out, ref_lse, BF16_OUT, BF16_LSE,
                 "selective reuse result")
    full_ref = oracle.merge(o_t1, l_t1)
    check_states(f_out[:, heads][:, :, rs], f_lse[:, heads][:, :, rs], full_ref[0], full_ref[1], BF16_OUT,
                 BF16_LSE, "full attention t+1")
    # weights at the anchor and at the reuse step against the oracle on the GPU's LSE
    w_ref, s_ref = oracle.contribution(runner.state_lse.reshape(w.P, -1).cpu().numpy(), Sq)
    assert np.abs(runner.anchor_weights.cpu().double().numpy() - w_ref).max() <= F32_TOL
    assert np.abs(runner.anchor_scores.cpu().double().numpy() - s_ref).max() <= F32_TOL
    w5, s5 = oracle.contribution(runner.step_lse.reshape(len(w.near) + 1, -1).cpu().numpy(), Sq)
    assert np.abs(runner.step_scores.cpu().double().numpy() - s5).max() <= F32_TOL
    # reuse error against full attention: reported; the near partitions hold most of the mass
    mse = torch.mean((r_out - f_out) ** 2).item()
    mean_w = runner.anchor_scores.mean(0).cpu().numpy()
    note(f"selective reuse: MSE vs full attention {mse:.3e}; near weight {mean_w[w.near].sum():.3f}")
    assert mean_w[w.near].sum() > 0.5
    assert mse < 1e-2
    # planner statistics at full size, against the oracle applied to the GPU's own states
    eps = to_dev(torch.tensor([1e-4], dtype=torch.float32))
    runner.plan_anchor()
    plan = runner.plan_step(w.local, 4, eps, 0.5)
    torch.cuda.synchronize()
    n_ref = np.array([oracle.planner.state_norm(runner.state_out[i].view(1, -1).cpu().numpy())[0]
                      for i in range(w.P)])
    np.testing.assert_allclose(runner.anchor_norms.cpu().double().numpy(), n_ref, rtol=NORM_RTOL, atol=0)
    fresh = runner.step_out[runner.near.index(w.local)].view(1, -1).cpu().numpy()
    d_ref = oracle.planner.state_norm(fresh, runner.state_out[w.local].view(1, -1).cpu().numpy())[0]
    np.testing.assert_allclose(runner.local_drift.cpu().double().numpy(), [d_ref], rtol=NORM_RTOL, atol=0)
    _, gw_ref = oracle.contribution(runner.state_lse.reshape(w.P, -1).cpu().numpy(), runner.rows)
    assert np.abs(runner.global_weights.cpu().double().numpy() - gw_ref).max() <= F32_TOL
    ref = oracle.planner.planner(runner.anchor_norms.cpu().numpy(), float(runner.local_drift.item()),
                                 runner.global_weights.view(-1).cpu().numpy(), w.local, 4, 1e-4, 0.5)
    np.testing.assert_allclose(plan["ase"].cpu().double().numpy(), ref["ase"], rtol=PLAN_RTOL, atol=0)
    gpu_ase = plan["ase"].cpu().double().numpy()
    assert np.array_equal(plan["compute"].cpu().numpy(),
                          oracle.planner.decide(gpu_ase, w.local, 4, float(np.float32(1e-4))))
    alpha = plan["alpha"].cpu().numpy()
    note(f"planner: local drift {runner.local_drift.item():.4g}, alpha near/far "
         f"{alpha[w.near].mean():.3f}/{np.delete(alpha, w.near).mean():.3f}, "
         f"group errors {np.array2string(gpu_ase, precision=2)}, compute {plan['compute'].cpu().numpy().tolist()}")


def test_full_size_long_video_fp8(reuse_workload):
    """Long-video anchor shape (32 partitions of 3840, D = 128) with fp8 q/k, as bench.py times it."""
    w = reuse_workload
    note(f"full size fp8 workload: {w.name}")
    q8, qs = inputs.quantize_fp8(to_dev(w.q))
    k8, ks = inputs.quantize_fp8(to_dev(w.k))
    w.v_dev = to_dev(w.v)
    fp8_full_size_check(w, q8, k8, qs, ks, [0, 11, 23], list(range(w.Sq)), "long video fp8")
    del w.v_dev


@pytest.mark.parametrize("near_group", [None, 2])
def test_full_size_grouped_selective_reuse(reuse_workload, reuse_reference, near_group):
    """The selective-reuse step with grouped launches at full size (every row of three heads): the
    anchor composes the far partitions in groups of 4 inside the attention launch, the next step
    folds the cached state into the near partitions' composed state (in one group, or in groups of
    two and then as_merge)."""
    w = reuse_workload
    note(f"full size grouped selective reuse, near_group={near_group}")
    runner = SelectiveReuse(w.B, w.H, w.Sq, w.D, w.ranges, w.near, DEV, w.scale)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    runner.anchor_grouped(q, k, v, far_group=4)
    del q, k, v
    r_out, r_lse = runner.step_grouped(to_dev(w.q1), to_dev(w.k1), to_dev(w.v1), near_group=near_group)
    torch.cuda.synchronize()
    o_t, l_t, o_t1, l_t1 = reuse_reference
    heads, rs = REUSE_HEADS, list(range(w.Sq))
    ref_out, ref_lse, c_out, c_lse = oracle.selective_reuse(o_t, l_t, o_t1, l_t1, w.near)
    check_states(runner.cached_out[:, heads][:, :, rs], runner.cached_lse[:, heads][:, :, rs], c_out, c_lse,
                 BF16_OUT, BF16_LSE, "grouped cached state")
    check_states(r_out[:, heads][:, :, rs], r_lse[:, heads][:, :, rs], ref_out, ref_lse, BF16_OUT, BF16_LSE,
                 "grouped reuse result")
    # every partition's LSE at the anchor, in the grouped order, and the near ones at the next step
    order, _ = runner.grouped_layout(4)
    got = runner.state_lse[:, :, heads].cpu().double().numpy()
    assert np.abs(got - l_t[order]).max() <= BF16_LSE
    got1 = runner.step_lse[:len(w.near), :, heads].cpu().double().numpy()
    assert np.abs(got1 - l_t1[w.near]).max() <= BF16_LSE


def test_prepared_launches_repeat_the_plain_calls_bitwise():
    """prepare_partition_attn / prepare_merge: arguments marshalled once, the same C calls; every
    repeated launch gives the plain call's result bit for bit."""
    w = inputs.small_case(31, 1, 2, 300, 1000, 128, RAGGED)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    note("prepared launches: partition_attn D=128 B=1 H=2 Sq=300 P=7, then a 7-way merge")
    out, lse = N.partition_attn(q, k, v, w.ranges, w.scale)
    launch, p_out, p_lse = N.prepare_partition_attn(q, k, v, w.ranges, w.scale)
    m_out, m_lse = N.merge(list(out), list(lse))
    mlaunch, pm_out, pm_lse = N.prepare_merge(list(out), list(lse))
    for _ in range(3):
        p_out.zero_()
        pm_out.zero_()
        launch()
        mlaunch()
        torch.cuda.synchronize()
        assert torch.equal(p_out, out) and torch.equal(p_lse, lse)
        assert torch.equal(pm_out, m_out) and torch.equal(pm_lse, m_lse)
