"""Pin of the oracle's decoder layer against a textbook layer written directly
with numpy fp64 matrix products from the full weight matrices (keeps of 1),
and against masked dense products and brute-force selections (keeps < 1)."""
import math

import numpy as np
import pytest

import oracle
from activation_kv_cache_amd import inputs as gen

DIMS = gen.TINY


def _f(a):
    return oracle.bf16_to_f64(a)


def _b(a):
    return oracle.f64_to_bf16(a)


def _textbook_layer(h, W, K, V, n, r_p, r_kv, sinks, window):
    d, H, Hkv, D, dff = DIMS["d"], DIMS["n_heads"], DIMS["n_kv_heads"], DIMS["head_dim"], DIMS["d_ff"]
    G = H // Hkv

    def norm(x, g):
        xv = _f(x)
        return _b(xv / np.sqrt(np.mean(xv ** 2) + 1e-5) * _f(g))

    def topk_mask(x, r):
        if r >= 1:
            return np.ones(x.size, bool)
        k = int(np.floor(r * x.size + 0.5))
        order = np.argsort(-(x & 0x7FFF).astype(np.int64), kind="stable")
        m = np.zeros(x.size, bool)
        m[order[:k]] = True
        return m

    def mv(wt, x, r):
        xv = _f(x) * topk_mask(x, r)
        return _f(wt).T @ xv

    def rot(v, nh):
        v = v.reshape(nh, D)
        i = np.arange(D // 2)
        z = (v[:, :D // 2] + 1j * v[:, D // 2:]) * np.exp(1j * (n - 1) * 500000.0 ** (-2.0 * i / D))
        return np.concatenate([z.real, z.imag], axis=1)

    x1 = norm(h, W["g1"])
    qkv = mv(W["qkv"], x1, r_p)
    q = _b(rot(qkv[:H * D], H))
    k = _b(rot(qkv[H * D:H * D + Hkv * D], Hkv))
    v = _b(qkv[H * D + Hkv * D:].reshape(Hkv, D))
    K = K.copy()
    V = V.copy()
    K[:, n - 1] = k
    V[:, n - 1] = v
    if r_kv < 1:
        summ = np.stack([oracle.kv_summary(K[g], n) for g in range(Hkv)])
        lists = oracle.kv_select(q, summ, n, H, Hkv, r_kv, sinks, window)
    else:
        lists = np.tile(np.arange(n), (Hkv, 1))
    a = np.zeros((H, D))
    for j in range(H):
        rows = lists[j // G]
        z = _f(K[j // G, rows]) @ _f(q[j]) / math.sqrt(D)
        p = np.exp(z - z.max())
        a[j] = p @ _f(V[j // G, rows]) / p.sum()
    a = _b(a.reshape(-1))
    h1 = _b(_f(h) + mv(W["o"], a, r_p))
    x2 = norm(h1, W["g2"])
    m = topk_mask(x2, r_p)
    gt = _f(W["gate"]).T @ (_f(x2) * m)
    up = _f(W["up"]).T @ (_f(x2) * m)
    f = _b(gt / (1 + np.exp(-gt)) * up)
    h2 = _b(_f(h1) + mv(W["down"], f, r_p))
    return {"x1": x1, "q": q, "k": k, "v": v, "a": a, "h_mid": h1, "x2": x2, "hff": f, "h_out": h2}


@pytest.mark.parametrize("r_p,r_kv", [(1.0, 1.0), (0.5, 1.0), (1.0, 0.3), (0.5, 0.3)])
def test_layer_matches_textbook(r_p, r_kv):
    n, n_cap, sinks, window, S = 2048, 2064, 4, 128, 8
    W = gen.layer_weights(0, DIMS)
    K, V = gen.kv_cache(0, DIMS, n_cap, 0.02)
    h = gen.normal_bf16(0, "h0", DIMS["d"])
    summ = np.zeros((DIMS["n_kv_heads"], n_cap // 16, DIMS["head_dim"], 2), np.uint16)
    for g in range(DIMS["n_kv_heads"]):
        s = oracle.kv_summary(K[g], n - 1)
        summ[g, :s.shape[0]] = s
    ref = _textbook_layer(h, W, K, V, n, r_p, r_kv, sinks, window)
    Ko, Vo, so = K.copy(), V.copy(), summ.copy()
    got = oracle.decode_layer(h, W, Ko, Vo, so, n, DIMS, r_p, r_kv, sinks, window, S)
    for name in ("x1", "q", "k", "v"):
        assert np.array_equal(got[name].reshape(-1), ref[name].reshape(-1)), name
    for name in ("a", "h_mid", "x2", "hff", "h_out"):
        g64, r64 = _f(got[name]).reshape(-1), _f(ref[name]).reshape(-1)
        rel = np.linalg.norm(g64 - r64) / max(np.linalg.norm(r64), 1e-30)
        assert rel < 2e-3, (name, rel)
    # the cache got the new row and the last block's summary covers it
    assert np.array_equal(Ko[:, n - 1], got["k"]) and np.array_equal(Vo[:, n - 1], got["v"])
    for g in range(DIMS["n_kv_heads"]):
        assert np.array_equal(so[g, (n - 1) // 16], oracle.kv_summary(Ko[g], n)[(n - 1) // 16])
    if r_p < 1:
        assert got["idx_qkv"].size == oracle.channel_keep(r_p, DIMS["d"])
        assert got["idx_down"].size == oracle.channel_keep(r_p, DIMS["d_ff"])
    if r_kv < 1:
        assert got["idx_kv"].shape == (DIMS["n_kv_heads"], 612)


def test_layer_teacher_forcing_replaces_inputs():
    n, n_cap, S = 256, 256, 4
    W = gen.layer_weights(1, DIMS)
    K, V = gen.kv_cache(1, DIMS, n_cap, 0.02)
    summ = np.stack([oracle.kv_summary(K[g], n) for g in range(DIMS["n_kv_heads"])])
    h = gen.normal_bf16(1, "h0", DIMS["d"])
    base = oracle.decode_layer(h, W, K.copy(), V.copy(), summ.copy(), n, DIMS, 0.5, 1.0, 4, 16, S)
    x1 = base["x1"].copy()
    x1[:10] = 0
    forced = oracle.decode_layer(h, W, K.copy(), V.copy(), summ.copy(), n, DIMS, 0.5, 1.0, 4, 16, S,
                                 forced={"x1": x1})
    assert np.array_equal(forced["x1"], base["x1"])          # own value is still reported
    assert not np.array_equal(forced["idx_qkv"], base["idx_qkv"])
    assert not np.any(np.isin(np.arange(10), forced["idx_qkv"]))
