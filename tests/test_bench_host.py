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


def test_snap_t_sel_matches_library(bc):
    for r_kv in (0.3, 0.5, 1.0):
        pol = bc.policy(r_kv, bench.SINKS, bench.WINDOW)
        for n in [1, 5, 1000, 1040, 2048, 4096, 6144, 32768, 65536 + 7, 131072]:
            assert bench.snap_t_sel(n, r_kv) == bc.bc_kv_snap_t_sel(n, pol), (n, r_kv)


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


def synthetic_full_record():
    """A full record shaped like a default run's: 12 cells, the kernel table,
    a 41-context sweep of 10 modes with 6 crossing pairs, the cpu baseline."""
    cells = []
    for n in (2048, 8192, 32768, 131072):
        cells.append({"r_p": 1.0, "r_kv": 1.0, "context": n, "kv_policy": "dense", "step_us": 5519.5,
                      "frac_hbm": 0.7301, "layer_us": 175.12, "speedup_vs_dense": 1.0})
    for n in (2048, 131072):
        for r_p, r_kv, pol in ((0.5, 1.0, "dense"), (1.0, 0.3, "scored"), (0.5, 0.3, "scored"),
                               (1.0, 0.3, "window")):
            cells.append({"r_p": r_p, "r_kv": r_kv, "context": n, "kv_policy": pol, "step_us": 3973.1,
                          "frac_hbm": 0.6401, "layer_us": 120.55, "speedup_vs_dense": 1.395})
    ctx = [2048] + [4096 * i for i in range(1, 41)]
    pairs = {}
    for mp, mk, r_p, r_kv in bench.PAIRS:
        key = f"{r_p}/{r_kv}" + (" sel" if bench.SWEEP_MODES[mk][2] else "")
        pairs[key] = {"n_star_k": 74.29, "n_star_ext_k": 81.6, "measured_k": 79.01, "pred_k": 81.3,
                      "measured_interval": {"resamples": 256, "no_crossing": 0, "level": 0.95, "lo_k": 78.71,
                                            "hi_k": 79.6}}
    return {
        "metric": bench.METRIC, "value": 5836.1, "unit": "GB/s", "n_gpus": 1, "steps": 20, "warmup": 5,
        "ms_per_step": 5.5195, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: random-init N(0,0.02) weights of Llama-3.1-8B shape, N(0,1) pre-filled KV cache",
        "config": {"workload": "dense decode step of one sequence at Llama-3.1-8B dims: 32 layers + LM head, "
                               "context 131072, r_p=1, r_kv=1", "context": 131072, "r_p": 1.0, "r_kv": 1.0,
                   "layers": 32, "batch": 1},
        "roofline": {"bound": "hbm", "kernel": "k_attn_partial (bc_splitk_attn_partial), dense, one layer",
                     "achieved": 6301.2, "peak": 8000.0, "unit": "GB/s", "frac": 0.7877,
                     "traffic": 537803776, "launch_us": 85.29, "bytes_per_launch": 537403392, "splits": 32},
        "read_probe": {"gbs": 7050.1, "frac_of_peak": 0.8813, "attention_frac_of_probe": 0.9012, "us": 76.1},
        "gemv_roofline": {"dense": {"frac": 0.8012}, "r_p_0.5": {"frac": 0.7055}},
        "cells": cells,
        "kernels": ([{"kernel": f"k{i}", "us": 1.0 * i} for i in range(40)]
                    + [{"kernel": f"gemv {w} r_p={rp}", "us": 10.0, "gbs": 4321.0}
                       for w in ("w_qkv", "w_o", "w_gu", "w_down") for rp in ("1.0", "0.7", "0.5")]
                    + [{"kernel": k, "context": n, "us": 30.0, "gbs": 5555.0, "probe_gbs": 6666.0,
                        "frac_of_probe": 0.8333}
                       for k in ("attn_partial dense", "attn_partial r_kv=0.3", "attn_partial r_kv=0.5")
                       for n in (2048, 8192, 32768, 131072)]),
        "crossover": {"contexts": ctx, "pairs": pairs,
                      "speedup": {m: [1.2345] * len(ctx) for m in bench.SWEEP_MODES if m != "dense"},
                      "step_us": {m: [1234.5] * len(ctx) for m in bench.SWEEP_MODES}},
        "composed": {"summary": {str(n): {f"{a}/{b}": [1.2345, 1.8765] for a, b in grid}
                                 for n, grid in bench.COMPOSED_GRID.items()}},
        "cpu_baseline": {"value": 1.5612, "unit": "GB/s", "cores": 16, "kind": "oracle", "cpu_model": "x" * 40,
                         "sample": "one of the 32 decoder layers of the dense 131072-token step (weights 436 MB + "
                                   "KV 537 MB), fp64 oracle, 16 run(s) in 10.1s; GB/s = that layer's algorithmic "
                                   "bytes / oracle time"},
    }


def test_compact_record_fits_and_parses():
    import json
    full = synthetic_full_record()
    full_len = len(json.dumps(full))
    line = bench.compact_record(full)
    assert len(line.encode()) <= bench.COMPACT_LIMIT < full_len
    rec = json.loads(line)
    # each GEMV's and the attention's fraction of peak sits beside the 70% target
    kf = rec["kernel_frac"]
    assert kf["target"] == 0.7
    for rp in ("1.0", "0.5"):
        assert set(kf[f"gemv_r_p_{rp}"]) == {"qkv", "o", "gu", "down"}
        assert kf[f"gemv_r_p_{rp}"]["o"] == round(4321.0 / bench.HBM_PEAK_GBS, 3)
    assert kf["attn"]["kv0.3@131072"] == [round(5555.0 / bench.HBM_PEAK_GBS, 3), 0.8333]
    assert "gemv_r_p_0.7" not in kf and not any("0.5@" in k for k in kf["attn"])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "dtype", "config",
              "roofline", "cpu_baseline"):
        assert k in rec, k
    assert rec["roofline"]["frac"] == 0.7877 and rec["roofline"]["traffic"] == 537803776
    assert rec["cpu_baseline"]["cores"] == 16 and rec["cpu_baseline"]["kind"] == "oracle"
    # the default run's summaries fit whole
    assert len(rec["cells"]) == 12 and len(rec["crossings_k"]) == len(bench.PAIRS)
    assert rec["composed"]["131072"]["0.5/0.3"] == [1.2345, 1.8765] and len(rec["composed"]["32768"]) == 4
    assert "\n" not in line


def test_compact_record_drops_summaries_before_the_headline():
    import json
    full = synthetic_full_record()
    full["cells"] = full["cells"] * 20          # far more cells than fit
    rec = json.loads(bench.compact_record(full))
    assert "cells" not in rec and rec["roofline"]["frac"] == 0.7877 and "cpu_baseline" in rec
    assert len(bench.compact_record(full).encode()) <= bench.COMPACT_LIMIT


@pytest.mark.parametrize("mp,mk,r_p,r_kv", bench.PAIRS)
def test_prediction_from_a_separate_calibration_grid(mp, mk, r_p, r_kv):
    """The prediction fitted on the coarse calibration contexts (a separate
    sweep) agrees with the one fitted on the crossover grid when the step
    times follow bytes / BW + per-mode constants exactly."""
    costs = {"dense": 250.0, mp: 700.0, mk: 520.0}
    fine = synthetic_times(6500.0, costs)
    ctx = bench.CALIB_CONTEXTS
    coarse = {m: np.array([bench.mode_bytes(m, n) / 6500e3 + costs.get(m, 0.0) for n in ctx])
              for m in ("dense", mp, mk)}
    p_fine = bench.predicted_crossing_k(CTX, fine, mp, mk)
    p_coarse = bench.predicted_crossing_k(ctx, coarse, mp, mk)
    assert p_coarse[0] == pytest.approx(p_fine[0], abs=1e-6)
    assert p_coarse[2] == pytest.approx(700.0, abs=1e-3) and p_coarse[3] == pytest.approx(520.0, abs=1e-3)


def test_step_pmc_summary_on_synthetic_counters(tmp_path):
    """The whole-step byte sum keeps only the dispatches after the marker,
    divides by the number of steps and scales by the copy calibration."""
    def write(path, rows):
        with open(path, "w") as fh:
            fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for d, k, v in rows:
                fh.write(f'{d},"{k}",X,{v}\n')
    # setup dispatches, the begin marker, 2 steps of two kernels each, the
    # end marker; a second mode's setup, its markers around one step of one
    # kernel
    fetch = [(1, "k_pack_tiles", 9e9), (2, "void bc::(anonymous namespace)::k_stream_read(uint4 const*)", 2048.0),
             (3, "void bc::(anonymous namespace)::k_gemv<1, 0, 4>(bc::GemvParams)", 1000.0),
             (4, "k_attn_partial<128, 4, 1, 0>(...)", 500.0),
             (5, "void bc::(anonymous namespace)::k_gemv<1, 0, 4>(bc::GemvParams)", 1000.0),
             (6, "k_attn_partial<128, 4, 1, 0>(...)", 500.0),
             (7, "k_stream_read(uint4 const*)", 2048.0), (8, "k_kv_compact", 5e9),
             (9, "k_stream_read(uint4 const*)", 2048.0), (10, "k_gemv<3, 0, 4>(...)", 300.0),
             (11, "k_stream_read(uint4 const*)", 2048.0)]
    write_ = [(d, k, v / 10) for d, k, v in fetch]
    write(tmp_path / "f.csv", fetch)
    write(tmp_path / "w.csv", write_)
    # the copy run fills its source first; only the copy dispatches count
    write(tmp_path / "cf.csv", [(1, "fill", 7.0), (2, "__amd_rocclr_copyBuffer", 512.0),
                                (3, "__amd_rocclr_copyBuffer", 512.0)])      # 1 MiB copy: fetch factor 0.5
    write(tmp_path / "cw.csv", [(1, "fill", 7.0), (2, "__amd_rocclr_copyBuffer", 1024.0)])     # write factor 1.0
    r, r2 = bench.step_pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                                   str(tmp_path / "cw.csv"), "dense:2048:2+proj0.5:2048:1", str(1 << 20))
    assert r2["fetch_bytes"] == round(300 * 1024 / 0.5) and list(r2["fetch_by_kernel"]) == ["k_gemv<3, 0, 4>"]
    assert r["copy_factors"] == {"fetch": 0.5, "write": 1.0}
    assert r["fetch_bytes"] == round(1500 * 1024 / 0.5)
    assert r["write_bytes"] == round(150 * 1024)
    assert r["measured_bytes"] == r["fetch_bytes"] + r["write_bytes"]
    assert set(r["fetch_by_kernel"]) == {"k_gemv<1, 0, 4>", "k_attn_partial<128, 4, 1, 0>"}
    assert r["algorithmic_bytes"] == bench.step_bytes(2048, 1.0, 1.0, *bench.kv_plan(2048, 1.0))


def test_attn_pmc_summary_on_synthetic_counters(tmp_path):
    """The attention kernel's bytes per launch: the mean over its dispatches
    of each counter, scaled by the copy calibration, against its algorithmic
    bytes, keyed to the kernel's code."""
    def write(path, rows):
        with open(path, "w") as fh:
            fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for d, k, v in rows:
                fh.write(f'{d},"{k}",X,{v}\n')
    att = "void bc::(anonymous namespace)::k_attn_partial<128, 4, 0, 0>(bc::AttnParams)"
    write(tmp_path / "f.csv", [(1, "k_fill", 9e9), (2, att, 262000.0), (3, att, 262400.0)])
    write(tmp_path / "w.csv", [(1, "k_fill", 9e9), (2, att, 570.0), (3, att, 580.0)])
    write(tmp_path / "cf.csv", [(1, "fill", 7.0), (2, "__amd_rocclr_copyBuffer", 512.0)])      # 1 MiB: 0.5
    write(tmp_path / "cw.csv", [(1, "fill", 7.0), (2, "__amd_rocclr_copyBuffer", 1024.0)])     # 1.0
    r = bench.attn_pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                               str(tmp_path / "cw.csv"), "131072", str(1 << 20))
    assert r["dispatches_averaged"] == 2 and r["fetch_size_kib_per_dispatch"] == 262200.0
    assert r["traffic_bytes_per_launch"] == round(262200.0 * 1024 / 0.5 + 575.0 * 1024)
    assert r["algorithmic_bytes_per_launch"] == 537403392
    assert r["kernel_source_hash"] == bench.kernel_source_hash() and r["context"] == 131072


def test_code_text_ignores_comments_and_white_space(tmp_path):
    """The counter summaries are keyed to the kernels' code: an edit of a
    comment keeps them valid, an edit of code (or of a string) does not."""
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text('int f(int x) {  // add one\n  return x + 1; /* done */\n}\nconst char* s = "a // b";\n')
    b.write_text('// another comment\nint f(int x) {\n    return x + 1;\n}\n/* x */ const char* s = "a // b";\n')
    c.write_text('int f(int x) {  // add one\n  return x + 2;\n}\nconst char* s = "a // b";\n')
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert '"a // b"' in bench.code_text(a)


def test_phase_clock_launch_reads_the_stamps():
    """One GEMV launch of two work-groups with known stamps: spans from the
    real-time counter (10 ns), phases from the shader clock at its measured
    rate (here 2000 MHz: 20 shader ticks per real-time tick)."""
    import numpy as np
    clk = np.zeros(64, dtype=np.int64)
    for g, (start, xcc) in enumerate(((1000, 0), (1010, 1))):
        e = clk[16 + 16 * g: 32 + 16 * g]        # slice at entry 16
        e[0], e[1] = start, start + 500          # 5 us of real time
        e[2] = 20 * start                        # shader clock, 2000 MHz
        e[3] = e[2] + 2000                       # inputs after 1 us
        e[4] = e[2] + 3000
        e[11] = e[2] + 6000                      # prologue 3 us
        e[12] = e[11] + 2000 * 1 + 4000 * g      # row loop 1 or 3 us
        e[13] = e[2] + 10000                     # 5 us in all
        e[14] = xcc
    launch = (1, 2 | (0 << 8), 14336, 4096, 7168, 2, 16)
    rec = bench.phase_clock_launch(launch, clk)
    assert rec["mhz"] == 2000
    assert rec["span_us"] == 5.1 and rec["skew_us"] == 0.1
    assert rec["kernel"].startswith("k_gemv sel/partial 14336x4096 k=7168")
    ph = rec["phases_us"]
    assert ph["inputs_arrived"] == 1.0 and ph["input_formed"] == 1.5 and ph["prologue"] == 3.0
    assert ph["row_loop"] == 2.0 and ph["total"] == 5.0 and ph["selected"] is None
    assert rec["xcc_wg_us"] == {0: 5.0, 1: 5.0}
