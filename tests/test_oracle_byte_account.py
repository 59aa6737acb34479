"""Pins of the oracle's byte account against every value the ByteCross README
prints (fixtures in tests/golden/byte_account.json, each with its section)."""
import json
import os

import pytest

from oracle import byte_account as ba

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "byte_account.json")))
M8B = ba.Model.from_config(GOLD["llama_3_1_8b_config"])


def _round(v, digits):
    return round(v, digits)


def test_from_config_matches_builtin():
    assert M8B == ba.LLAMA_31_8B
    assert M8B.head_dim == 128 and M8B.kv_dim == 1024


@pytest.mark.parametrize("case", GOLD["crossover_K"])
def test_crossover_printed(case):
    v = ba.crossover(M8B, case["rp"], case["rkv"]) / 1024
    assert _round(v, case["digits"]) == case["printed"]


@pytest.mark.parametrize("case", GOLD["crossover_ff_only_K"])
def test_crossover_ff_only_printed(case):
    v = ba.crossover(M8B, case["rp"], case["rkv"], ff_only=True) / 1024
    assert _round(v, case["digits"]) == case["printed"]


@pytest.mark.parametrize("case", GOLD["bound"])
def test_bound_printed(case):
    v = ba.bound(M8B, case["n"], rp=case["rp"], rkv=case["rkv"])
    assert _round(v, case["digits"]) == case["printed"]


@pytest.mark.parametrize("case", GOLD["crossover_batch_K"])
def test_crossover_batch_printed(case):
    v = ba.crossover_batch(M8B, case["union_keep"], case["rkv"], case["batch"]) / 1024
    assert _round(v, case["digits"]) == case["printed"]


@pytest.mark.parametrize("case", GOLD["matched_crossover_K"]["cases"])
def test_matched_crossover_printed(case):
    g = GOLD["matched_crossover_K"]
    proj = {float(k): v for k, v in g["proj"].items()}
    sel = {float(k): v for k, v in g["sel"].items()}
    v = ba.matched_crossover(M8B, proj, sel, case["budget"]) / 1024
    assert _round(v, g["digits"]) == case["printed"]


@pytest.mark.parametrize("row", GOLD["table1_K"]["rows"], ids=lambda r: r["model"])
def test_table1_rows(row):
    t = GOLD["table1_K"]
    m = ba.Model(n_layers=32, d=row["d"], d_ff=row["d_ff"], vocab=128256,
                 n_heads=row["n_heads"], n_kv_heads=row["n_kv_heads"])
    assert _round(ba.crossover(m, t["rp"], t["rkv"]) / 1024, 1) == row["n_star"]
    assert _round(ba.crossover(m, t["rp"], t["rkv"], ff_only=True) / 1024, 1) == row["n_star_ff"]


def test_bound_composition_is_pinned():
    """The printed 1.60 rules out the two neighbouring readings of B_total."""
    g = GOLD["not_pinned_composition"]
    n, rkv = g["n"], g["rkv"]
    kv = ba.kv_bytes(M8B, n)
    wp = ba.projection_bytes(M8B)
    no_head = (wp + kv) / (wp + kv - (1 - rkv) * kv)
    emb = ba.head_bytes(M8B)  # the embedding table has the LM head's shape
    with_emb = (wp + 2 * emb + kv) / (wp + 2 * emb + kv - (1 - rkv) * kv)
    assert round(no_head, 2) == g["without_head_rounds_to"]
    assert round(with_emb, 2) == g["with_embedding_rounds_to"]
    assert round(ba.bound(M8B, n, rkv=rkv), 2) == 1.60


def test_closed_form_invariants():
    # at n* the two savings are equal
    for rp, rkv in [(0.7, 0.3), (0.5, 0.3), (0.5, 0.5)]:
        n = ba.crossover(M8B, rp, rkv)
        assert abs((1 - rp) * ba.projection_bytes(M8B) - (1 - rkv) * ba.kv_bytes(M8B, n)) < 1e-3
    # keeps of 1 give no speedup; the composed bound exceeds each branch's
    assert ba.bound(M8B, 8192) == 1.0
    for n in (2048, 32768, 131072):
        both = ba.bound(M8B, n, 0.5, 0.3)
        assert both > ba.bound(M8B, n, rp=0.5) and both > ba.bound(M8B, n, rkv=0.3)
    # the crossover does not depend on layer count or vocab
    m2 = ba.Model(n_layers=7, d=4096, d_ff=14336, vocab=17, n_heads=32, n_kv_heads=8)
    assert abs(ba.crossover(m2, 0.5, 0.3) - ba.crossover(M8B, 0.5, 0.3)) < 1e-6
    # per-token KV bytes at 8B dims: 2 (K,V) * 32 layers * 1024 * 2 bytes
    assert ba.kv_bytes(M8B, 1) == 131072
    assert ba.layer_projection_params(M8B) == 218103808
