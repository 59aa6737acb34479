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
    return {m: np.array([bench.mode_bytes(m, n) / (bw_gbs * 1e3) + costs_us.get(m, 0.0) for n in CTX])
            for m in bench.SWEEP_MODES}


@pytest.mark.parametrize("mp,mk,r_p,r_kv", bench.PAIRS)
def test_prediction_without_costs_is_the_byte_crossing(mp, mk, r_p, r_kv):
    t = synthetic_times(6000.0, {"dense": 300.0, mp: 300.0, mk: 300.0})
    pred, bw, cp, ck = bench.predicted_crossing_k(CTX, t, mp, mk)
    assert bw == pytest.approx(6000.0, rel=1e-6)
    assert cp == pytest.approx(300.0, abs=1e-3) and ck == pytest.approx(300.0, abs=1e-3)
    # with equal costs the prediction is the step byte account's own crossing:
    # the first context where the KV branch moves no more bytes than the
    # projection branch (scanned token by token here)
    n = 1024
    while bench.mode_bytes(mk, n) > bench.mode_bytes(mp, n):
        n += 16
    assert pred == pytest.approx(n / 1024, abs=0.25)
    # a kv branch also writes and reads its index lists (16 B per selected
    # token and layer, 0.4% of the K and V bytes it keeps) and every budget
    # rounds to whole blocks, so the step's crossing lies up to ~2% above
    # n*_ext (Eq. 5 plus the summaries) for a kv branch and above n* for a
    # sel branch, never below it
    nx = bench.n_star_k(r_p, r_kv, ext=not bench.SWEEP_MODES[mk][2])
    assert nx - 0.1 <= pred <= nx * 1.025


@pytest.mark.parametrize("mp,mk,r_p,r_kv", bench.PAIRS)
def test_prediction_moves_by_the_cost_difference(mp, mk, r_p, r_kv):
    base = bench.predicted_crossing_k(CTX, synthetic_times(6000.0, {}), mp, mk)[0]
    extra_us = 400.0
    pred = bench.predicted_crossing_k(CTX, synthetic_times(6000.0, {mp: extra_us}), mp, mk)[0]
    # a fixed cost C on the projection branch is worth C * BW bytes of KV
    # savings: (1 - r_kv - 1/16) * KV(1) bytes per token
    D = bench.DIMS
    kv_per_token = 2 * 2 * D["n_layers"] * D["n_kv_heads"] * D["head_dim"]
    once = bench.SWEEP_MODES[mk][2]
    shift_k = extra_us * 1e-6 * 6000e9 / ((1 - r_kv - (0 if once else 1 / 16)) * kv_per_token) / 1024
    # (the step account's per-token KV saving is up to ~2% smaller than
    # Eq. 5's, for the index lists, so the shift is up to ~2% larger)
    assert shift_k - 0.3 <= base - pred <= shift_k * 1.025 + 0.3


@pytest.mark.parametrize("blocks", [1, 2, 3, 4, 5])
def test_block_resamples_enumerate_every_draw(blocks):
    d = bench.block_resamples(blocks)
    assert d.shape == (blocks ** blocks, blocks)
    assert d.min() == 0 and d.max() == blocks - 1
    assert len({tuple(r) for r in d}) == blocks ** blocks
    if blocks in (4, 5):   # the counts the paper quotes for four and five blocks
        assert len(d) == {4: 256, 5: 3125}[blocks]


def _pair_times(S_p, S_k):
    """Step times [blocks][contexts] with the given paired speedups against a
    dense time of 1000 us."""
    dense = np.full_like(S_p, 1000.0)
    return {"dense": dense, "p": dense / S_p, "k": dense / S_k}


def test_identical_blocks_give_a_point_interval():
    ctx = [4096 * i for i in range(1, 11)]
    n = np.array(ctx, float)
    S_k = np.tile(1.0 + n / 131072, (3, 1))
    S_p = np.tile(np.full(len(ctx), 1.2), (3, 1))
    speed, cross = bench.resample_intervals(_pair_times(S_p, S_k), ctx, [("x", "p", "k")])
    assert speed["p"]["lo"] == speed["p"]["hi"] == [1.2] * len(ctx)
    c = bench.crossing_k(ctx, list(S_p[0] - S_k[0]))
    assert cross["x"]["resamples"] == 27 and cross["x"]["no_crossing"] == 0
    assert cross["x"]["lo_k"] == cross["x"]["hi_k"] == round(c, 2)


def test_two_block_speedup_interval_by_hand():
    # draws (0,0) (0,1) (1,0) (1,1): resample means a, m, m, b with m = (a+b)/2;
    # the 2.5th percentile sits 0.075 of the way from a to m, the 97.5th 0.075 of the way from b to m
    a, b = 1.10, 1.30
    S = np.array([[a], [b]])
    speed, _ = bench.resample_intervals(_pair_times(S, S), [4096], [])
    m = (a + b) / 2
    assert speed["p"]["lo"][0] == pytest.approx(round(a + 0.075 * (m - a), 4), abs=1e-12)
    assert speed["p"]["hi"][0] == pytest.approx(round(b - 0.075 * (b - m), 4), abs=1e-12)


def test_crossing_interval_of_linear_differences():
    # block j: S_p - S_k = alpha * (c_j - n), so every resample crosses at the
    # mean of its drawn c_j (linear interpolation is exact on a line); block 3
    # never crosses inside the contexts, and resamples drawing only it are counted
    ctx = [4096 * i for i in range(1, 41)]
    n = np.array(ctx, float)
    c = np.array([40000.0, 52000.0, 61000.0, 1.0e6])
    alpha = 2e-7
    S_k = np.full((4, len(ctx)), 1.5)
    S_p = S_k + alpha * (c[:, None] - n[None, :])
    _, cross = bench.resample_intervals(_pair_times(S_p, S_k), ctx, [("x", "p", "k")])
    means = c[bench.block_resamples(4)].mean(axis=1)
    inside = means[means < ctx[-1]]
    assert cross["x"]["resamples"] == 256
    assert cross["x"]["no_crossing"] == int((means >= ctx[-1]).sum())
    lo, hi = np.percentile(inside / 1024, (2.5, 97.5))
    assert cross["x"]["lo_k"] == pytest.approx(round(lo, 2), abs=0.011)
    assert cross["x"]["hi_k"] == pytest.approx(round(hi, 2), abs=0.011)


@pytest.mark.parametrize("n", [2048, 8192, 32768, 131072])
@pytest.mark.parametrize("r_p,r_kv", [(1.0, 1.0), (0.5, 1.0), (1.0, 0.3), (0.7, 0.3), (0.5, 0.5)])
def test_byte_bound_matches_oracle(n, r_p, r_kv):
    from oracle import byte_account as ba
    assert bench.byte_bound(n, r_p, r_kv) == pytest.approx(ba.bound(ba.LLAMA_31_8B, n, rp=r_p, rkv=r_kv), rel=1e-12)


def test_window_baseline_bytes_leave_out_scoring():
    # the KV window keeps the same T tokens without summaries or index lists
    n, S = 131072, 32
    t = bench.kv_plan(n, 0.3)[0]
    scored = bench.layer_bytes(n, 1.0, 0.3, t, S)
    window = bench.layer_bytes(n, 1.0, 0.3, t, S, scored=False)
    D = bench.DIMS
    summaries = 2 * D["n_kv_heads"] * D["head_dim"] * 2 * (n // 16)
    assert scored - window == summaries + 2 * 4 * D["n_kv_heads"] * t


@pytest.mark.parametrize("u,r_kv,batch", [(0.92, 0.3, 4), (0.5, 0.3, 1), (0.97, 0.5, 2), (1.0, 0.3, 4)])
def test_batch_crossover_matches_oracle(u, r_kv, batch):
    from oracle import byte_account as ba
    want = ba.crossover_batch(ba.LLAMA_31_8B, union_keep=u, rkv=r_kv, batch=batch) / 1024
    assert bench.batch_crossover_k(u, r_kv, batch) == pytest.approx(want, rel=1e-12, abs=1e-12)
