"""The allocation-free contribution entry point (as_partition_contribution_noalloc), called
through the C ABI, against the allocating one (as_partition_contribution) on the same LSE:
two calls in a row, the second smaller, so the library's scratch still holds the first
call's partial sums when the second one runs."""
import numpy as np
import pytest
import torch

import oracle
from sequence_dit_amd import _native as N

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


def lse_block(seed, P, rows):
    g = np.random.default_rng(seed)
    lse = (g.standard_normal((P, rows)) * 6).astype(np.float32)
    lse[0, :5] = -np.inf
    lse[:, 7] = -np.inf   # a row where every partition is empty
    return lse


def allocating(lse, P, rows, rpg):
    w = torch.full((P, rows), float("nan"), device=DEV)
    s = torch.full((rows // rpg, P), float("nan"), device=DEV)
    need = N.contribution_workspace_size(P, rows, rpg)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    N.check(N.lib().as_partition_contribution(lse.data_ptr(), P, rows, rpg, w.data_ptr(), s.data_ptr(),
                                              ws.data_ptr(), ws.numel(), N._stream(lse)))
    return w, s


def allocation_free(lse, P, rows, rpg):
    w = torch.full((P, rows), float("nan"), device=DEV)
    s = torch.full((rows // rpg, P), float("nan"), device=DEV)
    N.check(N.lib().as_partition_contribution_noalloc(lse.data_ptr(), P, rows, rpg, w.data_ptr(), s.data_ptr(),
                                                      N._stream(lse)))
    return w, s


def test_noalloc_equals_allocating_entry_point_on_two_calls():
    # the long-video anchor's weights (32 partitions, 24 groups of 3840 rows), then a smaller call
    for seed, (P, rows, rpg) in enumerate(((32, 24 * 3840, 3840), (5, 1000, 250))):
        print(f"[gpu] noalloc contribution P={P} rows={rows} rows_per_group={rpg}", flush=True)
        lse_np = lse_block(seed + 1, P, rows)
        lse = torch.from_numpy(lse_np).to(DEV)
        w_ref, s_ref = allocating(lse, P, rows, rpg)
        w, s = allocation_free(lse, P, rows, rpg)
        torch.cuda.synchronize()
        # same kernels, same fixed reduction order: equal bit for bit
        assert torch.equal(w, w_ref) and torch.equal(s, s_ref)
        w_o, s_o = oracle.contribution(lse_np, rpg)
        assert np.abs(w.cpu().double().numpy() - w_o).max() <= 1e-5
        assert np.abs(s.cpu().double().numpy() - s_o).max() <= 1e-5


def test_noalloc_scores_only_and_weights_only():
    P, rows, rpg = 8, 777, 777
    lse_np = lse_block(9, P, rows)
    lse = torch.from_numpy(lse_np).to(DEV)
    w_ref, s_ref = allocating(lse, P, rows, rpg)
    s = torch.full((1, P), float("nan"), device=DEV)
    N.partition_contribution_noalloc(lse, rpg, scores=s)
    w = torch.full((P, rows), float("nan"), device=DEV)
    N.partition_contribution_noalloc(lse, rpg, weights=w)
    torch.cuda.synchronize()
    assert torch.equal(s, s_ref) and torch.equal(w, w_ref)
