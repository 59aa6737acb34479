"""Host-side pieces of bench.py: the KV plan replica against the library's
own budget and split rule, and the cost-aware crossing prediction (README
"Results", paper Table 2) on synthetic timings whose
answer is known."""
import numpy as np
import pytest

import bench
from activation_kv_cache_amd import binding


@pytest.fixture(scope="module")
def bc():
    return binding


@pytest.mark.parametrize("r_kv", [0.3, 0.5, 1.0])
def test_kv_plan_matches_library(bc, r_kv):
    pol = bc.policy(r_kv, bench.SINKS, bench.WINDOW)
    for n in [1, 5, 1000, 1040, 2048, 4096, 6144, 32768, 65536 + 7, 131072]:
        t_sel = bc.bc_kv_budget(n, pol)["t_sel"]
        S = bc.bc_attn_default_splits(t_sel, bench.DIMS["n_kv_heads"])
        assert bench.kv_plan(n, r_kv) == (t_sel, S), n


CTX = [2048] + [4096 * i for i in range(1, 33)]


def synthetic_times(bw_gbs, costs_us):
    """Step times that are exactly bytes / BW + a per-mode constant."""
    out = {}
    for m, (rp, rk) in bench.SWEEP_MODES.items():
        out[m] = np.array([bench.step_bytes(n, rp, rk, *bench.kv_plan(n, rk)) / (bw_gbs * 1e3) + costs_us.get(m, 0.0)
                           for n in CTX])
    return out


@pytest.mark.parametrize("mp,mk,r_p,r_kv", bench.PAIRS)
def test_prediction_without_costs_is_the_byte_crossing(mp, mk, r_p, r_kv):
    t = synthetic_times(6000.0, {"dense": 300.0, mp: 300.0, mk: 300.0})
    pred, bw, cp, ck = bench.predicted_crossing_k(CTX, t, mp, mk, r_p, r_kv)
    assert bw == pytest.approx(6000.0, rel=1e-6)
    assert cp == pytest.approx(300.0, abs=1e-3) and ck == pytest.approx(300.0, abs=1e-3)
    # with equal costs the prediction is the step byte account's own crossing:
    # the first context where the KV branch moves no more bytes than the
    # projection branch (scanned token by token here)
    def bytes_(n, rp, rk):
        return bench.step_bytes(n, rp, rk, *bench.kv_plan(n, rk))
    n = 1024
    while bytes_(n, 1.0, r_kv) > bytes_(n, r_p, 1.0):
        n += 16
    assert pred == pytest.approx(n / 1024, abs=0.25)
    # the KV branch also writes and reads its index lists (16 B per selected
    # token and layer, 0.4% of the K and V bytes it keeps) and the budget
    # rounds to whole blocks, so the step's crossing lies up to ~2% above
    # n*_ext (Eq. 5 plus the summaries), never below it
    nx = bench.n_star_k(r_p, r_kv, ext=True)
    assert nx - 0.1 <= pred <= nx * 1.025


@pytest.mark.parametrize("mp,mk,r_p,r_kv", bench.PAIRS)
def test_prediction_moves_by_the_cost_difference(mp, mk, r_p, r_kv):
    base = bench.predicted_crossing_k(CTX, synthetic_times(6000.0, {}), mp, mk, r_p, r_kv)[0]
    extra_us = 400.0
    pred = bench.predicted_crossing_k(CTX, synthetic_times(6000.0, {mp: extra_us}), mp, mk, r_p, r_kv)[0]
    # a fixed cost C on the projection branch is worth C * BW bytes of KV
    # savings: (1 - r_kv - 1/16) * KV(1) bytes per token
    D = bench.DIMS
    kv_per_token = 2 * 2 * D["n_layers"] * D["n_kv_heads"] * D["head_dim"]
    shift_k = extra_us * 1e-6 * 6000e9 / ((1 - r_kv - 1 / 16) * kv_per_token) / 1024
    # (the step account's per-token KV saving is up to ~2% smaller than
    # Eq. 5's, for the index lists, so the shift is up to ~2% larger)
    assert shift_k - 0.3 <= base - pred <= shift_k * 1.025 + 0.3
