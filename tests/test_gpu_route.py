"""GPU parity of moe_route_topk with the oracle router on inputs with many
equal logits, signed zeros, -inf and NaN entries, expert counts that are not
a multiple of the 64-lane wave, up to 32 selected experts and token counts
that span several workgroups.  Selection is compared exactly, weights within
fp32 exp rounding.  NaN sits only where at least k finite logits outrank it
in the same row (the oracle leaves a selected NaN undefined)."""
import numpy as np
import pytest

from tests.harness import log

pytestmark = pytest.mark.gpu

CASES = [  # (E, k, T)
    (8, 2, 5),
    (100, 8, 70),
    (128, 8, 255),  # 64 workgroups of four tokens, the last one ragged
    (256, 8, 33),
    (300, 8, 40),     # 257..512 experts: eight logits per lane
    (512, 16, 21),
    (1000, 32, 100),
]


def _logits(E, k, T, seed):
    rng = np.random.default_rng(seed)
    # a coarse grid of values, so most rows hold ties among their top k
    lg = (rng.integers(-6, 7, size=(T, E)) * 0.25).astype(np.float32)
    # some rows at most zero, so +0 and -0 are among the selected logits
    lg[3::11] = -np.abs(lg[3::11])
    zeros = rng.random((T, E)) < 0.05
    lg[zeros] = np.where(rng.random(zeros.sum()) < 0.5, np.float32(-0.0), np.float32(0.0))
    lg[rng.random((T, E)) < 0.03] = -np.inf
    # NaN only in rows where k finite logits stay
    nan = rng.random((T, E)) < 0.03
    for t in range(T):
        finite = np.isfinite(lg[t]) & ~nan[t]
        if finite.sum() < k + 1:
            nan[t] = False
    lg[nan] = np.nan
    # a few rows of one repeated value: the first k experts win
    lg[::17] = np.float32(0.5)
    return lg


def _oracle_route(lg, k):
    """The oracle's router with NaN read as -inf: the kernel's stated
    convention, and the oracle's order for every row built above."""
    from oracle.route import route_topk
    return route_topk(np.where(np.isnan(lg), np.float32(-np.inf), lg).astype(np.float32), k)


@pytest.mark.parametrize("E,k,T", CASES)
def test_route_topk_edges(E, k, T):
    import torch
    import routed_expert_execution_moe_amd as B
    log(f"route E={E} k={k} T={T}")
    cfg = B.config(1, E, k, 64, 64, "f32", "f32", n_slots=2, max_tokens=T, bw_pcie_mbps=1000,
                   bw_host_mbps=2000)
    stride = B.moe_expert_bytes(cfg)
    assert stride > 0, "config rejected"
    nbytes = E * stride
    pool = B.moe_host_pool_alloc(nbytes)
    ctx = None
    try:
        ctx = B.moe_create(cfg, pool, nbytes)
        dev = torch.device("cuda:0")
        for seed in (1, 2):
            lg = _logits(E, k, T, seed * 1000 + E)
            ids = torch.empty((T, k), dtype=torch.int32, device=dev)
            w = torch.empty((T, k), dtype=torch.float32, device=dev)
            B.moe_route_topk(ctx, torch.from_numpy(lg).to(dev), T, ids, w)
            torch.cuda.synchronize()
            ids_o, w_o = _oracle_route(lg, k)
            assert np.array_equal(ids.cpu().numpy(), ids_o), (E, k, T, seed)
            assert np.allclose(w.cpu().numpy(), w_o, rtol=2e-6, atol=1e-7), (E, k, T, seed)
            assert np.array_equal(ids_o[::17], np.broadcast_to(np.arange(k), ids_o[::17].shape))
    finally:
        if ctx:
            B.moe_destroy(ctx)
        B.moe_host_pool_free(pool)
