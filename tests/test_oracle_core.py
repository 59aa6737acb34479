"""Pins of the CPU oracle against what the mathematics fixes: closed forms,
library routines for special cases, brute force on tiny inputs, and
invariants chosen so that a dropped term, a wrong sign or index, or a
transposed operand fails at least one of them."""
import math

import numpy as np
import pytest
import torch

import oracle
from activation_kv_cache_amd import inputs as gen


# ----------------------------------------------------------------- bf16 codec
def test_bf16_codec_known_values():
    # 1.0, ties to even at 1 + 2^-8 (down) and 1 + 3*2^-8 (up), negative, subnormal, overflow
    vals = [1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 2.0 ** -133, 2.0 ** -133 * 1.5, 2.0 ** -133 * 2.5, 3.5e38, 0.0, -0.0]
    want = [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0001, 0x0002, 0x0002, 0x7F80, 0x0000, 0x8000]
    got = oracle.f64_to_bf16(np.array(vals))
    assert [int(v) for v in got] == want
    assert oracle.bf16_to_f64(np.array([0x3F80, 0xC020, 0x0001, 0x7F7F], np.uint16)).tolist() == [
        1.0, -2.5, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127]


def test_bf16_codec_matches_torch_rne():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(20000).astype(np.float32) * 10.0 ** g.integers(-30, 30, 20000),
                        g.standard_normal(1000).astype(np.float32) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)
    back = oracle.bf16_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


# --------------------------------------------------------- channel selection
def test_channel_keep_rounding():
    assert oracle.channel_keep(0.5, 4096) == 2048
    assert oracle.channel_keep(0.7, 4096) == 2867       # 2867.2
    assert oracle.channel_keep(0.7, 14336) == 10035     # 10035.2
    assert oracle.channel_keep(0.5, 1408) == 704
    assert oracle.channel_keep(1.0, 77) == 77
    assert oracle.channel_keep(0.0001, 77) == 1
    assert oracle.channel_keep(0.25, 6) == 2            # 1.5 + 0.5 = 2


def test_select_identity_and_all_equal():
    x = gen.normal_bf16(0, "sel/x", 300)
    assert np.array_equal(oracle.select_channels(x, 300), np.arange(300))
    same = np.full(100, 0x3F80, np.uint16)
    same[::2] |= 0x8000   # -1.0 and +1.0 tie on |x|
    assert np.array_equal(oracle.select_channels(same, 37), np.arange(37))


def test_select_hand_ladder():
    # |x| = 3, 1, 2, 3, 2, 1, 2 (signs mixed) ; k = 4 -> both 3s (0, 3) then the two lowest-index 2s (2, 4)
    vals = [3.0, -1.0, 2.0, -3.0, -2.0, 1.0, 2.0]
    x = gen.to_bf16_bits(np.array(vals, np.float32))
    assert oracle.select_channels(x, 4).tolist() == [0, 2, 3, 4]
    assert oracle.select_channels(x, 2).tolist() == [0, 3]
    assert oracle.select_channels(x, 6).tolist() == [0, 1, 2, 3, 4, 6]   # one |x|=1, the lower index
    # -0 and +0 tie
    z = np.array([0x8000, 0x0000, 0x8000], np.uint16)
    assert oracle.select_channels(z, 2).tolist() == [0, 1]


@pytest.mark.parametrize("n,k,levels", [(1408, 704, 5), (4096, 2867, 1000), (513, 1, 3), (64, 63, 2)])
def test_select_vs_numpy_stable_sort(n, k, levels):
    x = gen.tie_ladder_bf16(n, levels, 3, f"sel{n}")
    key = (x & 0x7FFF).astype(np.int64)
    order = np.argsort(-key, kind="stable")
    want = np.sort(order[:k])
    assert np.array_equal(oracle.select_channels(x, k), want)
    # the kept set dominates the dropped set in |x|
    vals = np.abs(oracle.bf16_to_f64(x))
    kept = np.zeros(n, bool)
    kept[want] = True
    if 0 < k < n:
        assert vals[kept].min() >= vals[~kept].max()


# --------------------------------------------------------------- sparse GEMV
def test_gemv_dense_is_matmul_and_masking_identity():
    wt = gen.normal_bf16(0, "g/w", (96, 40), 0.5)
    x = gen.normal_bf16(0, "g/x", 96)
    W = oracle.bf16_to_f64(wt).T          # W[o][i]
    xv = oracle.bf16_to_f64(x)
    y64, yb = oracle.sparse_gemv(wt, x)
    assert np.allclose(y64, W @ xv, rtol=1e-13, atol=1e-13)
    assert np.array_equal(yb, oracle.f64_to_bf16(W @ xv))
    idx = oracle.select_channels(x, 30)
    ys, _ = oracle.sparse_gemv(wt, x, idx)
    xm = np.zeros_like(xv)
    xm[idx] = xv[idx]
    assert np.allclose(ys, W @ xm, rtol=1e-13, atol=1e-13)
    # brute force, one output at a time, in list order
    for o in (0, 17, 39):
        acc = 0.0
        for i in idx:
            acc += W[o, i] * xv[i]
        assert ys[o] == acc


def test_gemv_empty_rows_and_transposition():
    # a non-square case catches a transposed operand
    wt = np.zeros((3, 5), np.uint16)
    wt[1, 4] = 0x3F80                   # W[4][1] = 1
    x = gen.to_bf16_bits(np.array([7.0, 2.0, 5.0], np.float32))
    y64, _ = oracle.sparse_gemv(wt, x)
    assert y64.tolist() == [0, 0, 0, 0, 2.0]
    y64, _ = oracle.sparse_gemv(wt, x, np.array([0, 2], np.int32))
    assert y64.tolist() == [0, 0, 0, 0, 0]


# --------------------------------------------------------------- layer glue
def test_rmsnorm_properties():
    x = gen.normal_bf16(0, "n/x", 512, 3.0)
    g = gen.to_bf16_bits(np.ones(512, np.float32))
    y = oracle.bf16_to_f64(oracle.rmsnorm(x, g, eps=0.0))
    assert abs(np.sqrt(np.mean(y ** 2)) - 1.0) < 4e-3
    xv = oracle.bf16_to_f64(x)
    assert np.array_equal(oracle.rmsnorm(x, g, eps=0.0), oracle.f64_to_bf16(xv / np.sqrt(np.mean(xv ** 2))))
    # scaling the input by a power of two changes nothing; the gain multiplies
    x4 = oracle.f64_to_bf16(xv * 4)
    assert np.array_equal(oracle.rmsnorm(x4, g, eps=0.0), oracle.rmsnorm(x, g, eps=0.0))
    g2 = gen.to_bf16_bits(np.full(512, 2.0, np.float32))
    assert np.array_equal(oracle.bf16_to_f64(oracle.rmsnorm(x, g2, 0.0)),
                          2 * oracle.bf16_to_f64(oracle.rmsnorm(x, g, 0.0)))


def test_rope_against_complex_rotation():
    D, Hn, pos, theta = 64, 3, 1234, 500000.0
    v = np.random.default_rng(2).standard_normal(Hn * D)
    got = oracle.rope(v, Hn, D, pos, theta).reshape(Hn, D)
    vv = v.reshape(Hn, D)
    i = np.arange(D // 2)
    z = (vv[:, :D // 2] + 1j * vv[:, D // 2:]) * np.exp(1j * pos * theta ** (-2.0 * i / D))
    assert np.allclose(got[:, :D // 2], z.real, atol=1e-12)
    assert np.allclose(got[:, D // 2:], z.imag, atol=1e-12)
    assert np.allclose(oracle.rope(v, Hn, D, 0), v)                   # position 0 is the identity
    assert np.allclose(np.linalg.norm(got), np.linalg.norm(v))       # a rotation


def test_swiglu_closed_form():
    g = np.array([0.0, 1.0, -2.0, 5.0])
    u = np.array([3.0, 2.0, 1.0, -1.0])
    want = g / (1 + np.exp(-g)) * u
    assert np.array_equal(oracle.swiglu(g, u), oracle.f64_to_bf16(want))
    assert oracle.swiglu(np.array([0.0]), np.array([9.0]))[0] == 0


# ------------------------------------------------------------ KV selection
def test_kv_summary_brute_force():
    k = gen.normal_bf16(0, "s/k", (70, 8))
    s = oracle.kv_summary(k, 53)          # 4 blocks; the last holds 5 tokens
    assert s.shape == (4, 8, 2)
    kv = oracle.bf16_to_f64(k)
    for b in range(4):
        blk = kv[16 * b:min(16 * b + 16, 53)]
        assert np.array_equal(oracle.bf16_to_f64(s[b, :, 0]), blk.min(0))
        assert np.array_equal(oracle.bf16_to_f64(s[b, :, 1]), blk.max(0))


def test_kv_budget_cases():
    b = oracle.kv_budget(2048, 0.3, 4, 128)
    assert (b["T_sel"], b["k_blk"], b["n_cand"], b["b_lo"]) == (612, 30, 119, 1)
    b = oracle.kv_budget(131072, 0.3, 4, 1024)
    assert (b["T_sel"], b["k_blk"], b["n_cand"]) == (39316, 2393, 8127)
    b = oracle.kv_budget(131072, 0.5, 4, 1024)
    assert (b["T_sel"], b["k_blk"]) == (65524, 4031)
    # T below sinks + window: a pure sinks + window list
    b = oracle.kv_budget(2048, 0.3, 4, 1024)
    assert (b["T_sel"], b["k_blk"], b["window"]) == (614, 0, 610)
    assert oracle.kv_budget(1000, 1.0, 4, 128)["T_sel"] == 1000


def _score64(qg, sb):
    q = oracle.bf16_to_f64(qg)
    mn = oracle.bf16_to_f64(sb[:, 0])
    mx = oracle.bf16_to_f64(sb[:, 1])
    return float(np.maximum(q * mx, q * mn).sum())


def test_block_score_rounding_and_bound():
    G, D = 4, 128
    rng = np.random.default_rng(5)
    for trial in range(20):
        qg = gen.to_bf16_bits(rng.standard_normal((G, D)).astype(np.float32))
        keys = gen.to_bf16_bits(rng.standard_normal((16, D)).astype(np.float32))
        sb = oracle.kv_summary(keys, 16)[0]
        s32 = oracle.block_score(qg, sb)
        s64 = _score64(qg, sb)
        t_abs = np.abs(np.maximum(oracle.bf16_to_f64(qg) * oracle.bf16_to_f64(sb[:, 1]),
                                  oracle.bf16_to_f64(qg) * oracle.bf16_to_f64(sb[:, 0]))).sum()
        assert abs(s32 - s64) <= 10 * 2.0 ** -24 * t_abs
        # upper bound of q_j . k_t summed over the group, for every token of the block
        kv = oracle.bf16_to_f64(keys)
        qv = oracle.bf16_to_f64(qg)
        for t in range(16):
            assert s64 >= float((qv @ kv[t]).sum()) - 1e-9
    # equality when all rows of the block are the same key
    row = gen.to_bf16_bits(rng.standard_normal(D).astype(np.float32))
    sb = oracle.kv_summary(np.tile(row, (16, 1)), 16)[0]
    assert abs(_score64(qg, sb) - float((oracle.bf16_to_f64(qg) @ oracle.bf16_to_f64(row)).sum())) < 1e-9


def test_block_score_exact_order_small():
    """With values chosen so float rounding matters, the oracle's order (per
    dim the heads' positive parts summed first, then one product pair per dim,
    pairs of 4 dims, then dim-groups by adjacent pairs) gives a sum that a
    per-head order would not."""
    G, D = 2, 4
    q = np.array([[2.0 ** 24, 0, 0, 0], [1, 1, 0, 0]], np.float32)
    k = np.array([1, 1, 0, 0], np.float32)
    summ = np.stack([k, k], axis=1)          # kmin = kmax
    s = oracle.block_score(gen.to_bf16_bits(q), gen.to_bf16_bits(summ))
    # P_0 = fl(2^24 + 1) = 2^24 (ties to even), P_1 = 1; t = (2^24, 1, 0, 0);
    # a = fl(2^24 + 1) + 0 = 2^24
    assert s == 2.0 ** 24
    # the exact bound is 2^24 + 2, which a per-head order (head 1 summed to 2
    # first) would also give
    assert abs(_score64(gen.to_bf16_bits(q), gen.to_bf16_bits(summ)) - (2.0 ** 24 + 2)) < 1e-9
    # the negative parts take the minima: q = -1 on a block with kmin = -3,
    # kmax = 5 contributes (-1) * (-3) = 3, the larger of -5 and 3
    q2 = np.array([[-1, 0, 0, 0]], np.float32)
    summ2 = np.array([[-3, 5], [0, 0], [0, 0], [0, 0]], np.float32)
    assert oracle.block_score(gen.to_bf16_bits(q2), gen.to_bf16_bits(summ2)) == 3.0


def _brute_kv_select(q, summ, n, H, Hkv, r_kv, sinks, window):
    bud = oracle.kv_budget(n, r_kv, sinks, window)
    G = H // Hkv
    out = []
    for g in range(Hkv):
        cands = list(range(bud["b_lo"], bud["b_lo"] + bud["n_cand"]))
        sc = [oracle.block_score(q[g * G:(g + 1) * G], summ[g, b]) for b in cands]
        order = sorted(range(len(cands)), key=lambda i: (-sc[i], cands[i]))
        chosen = sorted(cands[i] for i in order[:bud["k_blk"]])
        lst = list(range(bud["sinks"]))
        for b in chosen:
            lst += list(range(16 * b, 16 * b + 16))
        lst += list(range(n - bud["window"], n))
        out.append(lst)
    return np.array(out, np.int32)


@pytest.mark.parametrize("n,r_kv,sinks,window", [(2048, 0.3, 4, 128), (1000, 0.5, 4, 64),
                                                 (333, 0.2, 4, 16), (2048, 0.3, 4, 1024)])
def test_kv_select_brute_force_and_invariants(n, r_kv, sinks, window):
    H, Hkv, D = 8, 2, 64
    q = gen.normal_bf16(1, "ks/q", (H, D))
    K = gen.normal_bf16(1, "ks/k", (Hkv, 2048, D), 0.02)
    nb_cap = 2048 // 16
    summ = np.zeros((Hkv, nb_cap, D, 2), np.uint16)
    for g in range(Hkv):
        s = oracle.kv_summary(K[g], n)
        summ[g, :s.shape[0]] = s
    idx, scores = oracle.kv_select(q, summ, n, H, Hkv, r_kv, sinks, window, want_scores=True)
    assert np.array_equal(idx, _brute_kv_select(q, summ, n, H, Hkv, r_kv, sinks, window))
    bud = oracle.kv_budget(n, r_kv, sinks, window)
    assert idx.shape == (Hkv, bud["T_sel"])
    for g in range(Hkv):
        row = idx[g]
        assert np.all(np.diff(row) > 0) and row.min() >= 0 and row.max() < n
        assert set(range(bud["sinks"])) <= set(row.tolist())
        assert set(range(n - bud["window"], n)) <= set(row.tolist())


def test_kv_select_planted_block_and_dense():
    H, Hkv, D, n = 8, 2, 64, 2048
    q = gen.normal_bf16(2, "pl/q", (H, D))
    K = gen.normal_bf16(2, "pl/k", (Hkv, n, D), 0.02)
    qv = oracle.bf16_to_f64(q)
    planted = 57
    for g in range(Hkv):
        direction = qv[g * 4:(g + 1) * 4].sum(0)
        K[g, 16 * planted:16 * planted + 16] = oracle.f64_to_bf16(
            np.tile(direction / np.linalg.norm(direction), (16, 1)))
    summ = np.stack([oracle.kv_summary(K[g], n) for g in range(Hkv)])
    idx = oracle.kv_select(q, summ, n, H, Hkv, 0.02, 4, 16)   # budget: exactly 1 block
    assert oracle.kv_budget(n, 0.02, 4, 16)["k_blk"] == 1
    for g in range(Hkv):
        assert list(idx[g, 4:20]) == list(range(16 * planted, 16 * planted + 16))
    dense = oracle.kv_select(q, summ, n, H, Hkv, 1.0, 4, 16)
    assert np.array_equal(dense, np.tile(np.arange(n, dtype=np.int32), (Hkv, 1)))


@pytest.mark.parametrize("n,r_kv", [(2048, 0.3), (2051, 0.5), (40000, 0.3), (17, 0.3), (3, 0.5)])
def test_kv_window_policy_is_sinks_and_most_recent(n, r_kv):
    """A window at least as long as the context leaves no room for scored
    blocks: the kept set is the first min(4, T) tokens and the T - 4 most
    recent ones, T = floor(r_kv n + 1/2) (the sinks-plus-recent window of
    StreamingLLM that the paper's KV-window baseline keeps)."""
    H, Hkv, D = 8, 2, 64
    q = gen.normal_bf16(4, f"win/q{n}", (H, D))
    summ = np.zeros((Hkv, (n + 15) // 16, D, 2), np.uint16)
    bud = oracle.kv_budget(n, r_kv, 4, n)
    T = min(n, int(math.floor(r_kv * n + 0.5)))
    s = min(4, T)
    want = np.array(list(range(s)) + list(range(n - (T - s), n)), np.int32)
    assert bud["k_blk"] == 0 and bud["T_sel"] == T
    idx = oracle.kv_select(q, summ, n, H, Hkv, r_kv, 4, n)
    assert np.array_equal(idx, np.tile(want, (Hkv, 1)))


# ------------------------------------------------------------------ attention
def _softmax_attention(q, K, V, lst, H, Hkv):
    """Textbook softmax(q K^T / sqrt(D)) V over the listed tokens, numpy fp64."""
    D = q.shape[1]
    G = H // Hkv
    qv, Kv, Vv = (oracle.bf16_to_f64(a) for a in (q, K, V))
    out = np.zeros((H, D))
    for j in range(H):
        g = j // G
        rows = lst[g] if lst is not None else np.arange(K.shape[1])
        z = Kv[g, rows] @ qv[j] / math.sqrt(D)
        p = np.exp(z - z.max())
        out[j] = (p / p.sum()) @ Vv[g, rows]
    return out


@pytest.mark.parametrize("S", [1, 3, 8, 17])
def test_attention_any_split_equals_softmax(S):
    H, Hkv, D, n = 8, 2, 64, 300
    q = gen.normal_bf16(3, "at/q", (H, D))
    K = gen.normal_bf16(3, "at/k", (Hkv, n, D), 0.5)
    V = gen.normal_bf16(3, "at/v", (Hkv, n, D), 1.0)
    m, l, o = oracle.attn_partial(q, K, V, None, n, H, Hkv, S)
    out64, outb = oracle.attn_reduce(m, l, o)
    ref = _softmax_attention(q, K, V, None, H, Hkv)
    assert np.allclose(out64, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(outb, oracle.f64_to_bf16(ref))
    # per-split meaning: m is the max logit of the split
    c = -(-n // S)
    qv, Kv = oracle.bf16_to_f64(q), oracle.bf16_to_f64(K)
    for s in range(S):
        lo, hi = s * c, min(n, s * c + c)
        if lo < hi:
            assert abs(m[5, s] - (Kv[1, lo:hi] @ qv[5]).max() / 8.0) < 1e-12
        else:
            assert m[5, s] == -np.inf and l[5, s] == 0


def test_attention_lists_and_special_cases():
    H, Hkv, D, n = 8, 2, 64, 200
    q = gen.normal_bf16(4, "as/q", (H, D))
    K = gen.normal_bf16(4, "as/k", (Hkv, n, D), 0.5)
    V = gen.normal_bf16(4, "as/v", (Hkv, n, D), 1.0)
    ident = np.tile(np.arange(n, dtype=np.int32), (Hkv, 1))
    a1 = oracle.attn_reduce(*oracle.attn_partial(q, K, V, None, n, H, Hkv, 5))[0]
    a2 = oracle.attn_reduce(*oracle.attn_partial(q, K, V, ident, n, H, Hkv, 5))[0]
    assert np.array_equal(a1, a2)
    # a list: same as the textbook over those rows; permuting it changes only rounding
    rng = np.random.default_rng(0)
    lst = np.stack([np.sort(rng.choice(n, 77, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    a3 = oracle.attn_reduce(*oracle.attn_partial(q, K, V, lst, 77, H, Hkv, 4))[0]
    assert np.allclose(a3, _softmax_attention(q, K, V, lst, H, Hkv), atol=1e-12)
    perm = np.stack([rng.permutation(r) for r in lst]).astype(np.int32)
    a4 = oracle.attn_reduce(*oracle.attn_partial(q, K, V, perm, 77, H, Hkv, 4))[0]
    assert np.allclose(a3, a4, atol=1e-12)
    # q = 0: the mean of the listed value rows
    q0 = np.zeros_like(q)
    a5 = oracle.attn_reduce(*oracle.attn_partial(q0, K, V, lst, 77, H, Hkv, 3))[0]
    Vv = oracle.bf16_to_f64(V)
    for j in range(H):
        assert np.allclose(a5[j], Vv[j // 4, lst[j // 4]].mean(0), atol=1e-12)
    # a single token gives its value row
    one = np.array([[17], [150]], np.int32)
    a6 = oracle.attn_reduce(*oracle.attn_partial(q, K, V, one, 1, H, Hkv, 4))[0]
    assert np.array_equal(a6[0], Vv[0, 17]) and np.array_equal(a6[7], Vv[1, 150])
    # GQA grouping: query head j reads KV head j // (H/Hkv)
    K2 = K.copy()
    K2[1] = 0
    a7 = oracle.attn_reduce(*oracle.attn_partial(q, K2, V, None, n, H, Hkv, 2))[0]
    assert np.allclose(a7[:4], a1[:4]) and np.allclose(a7[4], Vv[1, :n].mean(0), atol=1e-12)


def test_attention_brute_force_tiny():
    H, Hkv, D, n, S = 2, 1, 4, 5, 2
    q = gen.to_bf16_bits(np.array([[1, 0, 0, 0], [0, 2, 0, 0]], np.float32))
    kk = np.zeros((1, n, D), np.float32)
    kk[0, :, 0] = [0, 1, 2, 3, 4]
    kk[0, :, 1] = [1, 0, 0, 0, 1]
    vv = np.zeros((1, n, D), np.float32)
    vv[0, :, 2] = [1, 2, 3, 4, 5]
    m, l, o = oracle.attn_partial(q, gen.to_bf16_bits(kk), gen.to_bf16_bits(vv), None, n, H, Hkv, S)
    # split 0 = tokens 0..2, split 1 = tokens 3..4; head 0 logits = k0 / 2
    assert m[0, 0] == 1.0 and m[0, 1] == 2.0
    assert abs(l[0, 0] - (math.exp(-1) + math.exp(-0.5) + 1)) < 1e-15
    assert abs(o[0, 1, 2] - (4 * math.exp(-0.5) + 5)) < 1e-14
    out64, _ = oracle.attn_reduce(m, l, o)
    w = np.exp(np.array([0, 1, 2, 3, 4]) / 2.0)
    assert abs(out64[0, 2] - (w @ np.array([1, 2, 3, 4, 5])) / w.sum()) < 1e-14
    w1 = np.exp(np.array([2, 0, 0, 0, 2]) / 2.0)
    assert abs(out64[1, 2] - (w1 @ np.array([1, 2, 3, 4, 5])) / w1.sum()) < 1e-14


def test_kv_compact_then_dense_attention_equals_list_attention():
    """The sel mode (README "Timing and quality on a GPU"): the selection
    gathered into a contiguous buffer and read densely is the attention over
    the index list -- the same sums in the same order -- and a planted row
    lands where its list position says."""
    H, Hkv, D, n, n_out = 8, 2, 64, 500, 160
    q = gen.normal_bf16(6, "kc/q", (H, D))
    K = gen.normal_bf16(6, "kc/k", (Hkv, n, D), 0.5)
    V = gen.normal_bf16(6, "kc/v", (Hkv, n, D), 1.0)
    rng = np.random.default_rng(6)
    t_sel = 150
    lst = np.stack([np.sort(rng.choice(n, t_sel, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    Kc, Vc = oracle.kv_compact(K, V, lst, n_out)
    assert Kc.shape == (Hkv, n_out, D) and not Kc[:, t_sel:].any() and not Vc[:, t_sel:].any()
    for S in (1, 4, 7):
        a_list = oracle.attn_partial(q, K, V, lst, t_sel, H, Hkv, S)
        a_comp = oracle.attn_partial(q, Kc, Vc, None, t_sel, H, Hkv, S)
        for x, y in zip(a_list, a_comp):
            assert np.array_equal(x, y)
    # head 1's 37th kept token is row lst[1][37] of the cache
    assert np.array_equal(Kc[1, 37], K[1, lst[1, 37]]) and np.array_equal(Vc[1, 37], V[1, lst[1, 37]])
    # the identity list copies the first rows
    ident = np.tile(np.arange(t_sel, dtype=np.int32), (Hkv, 1))
    Ki, Vi = oracle.kv_compact(K, V, ident, t_sel)
    assert np.array_equal(Ki, K[:, :t_sel]) and np.array_equal(Vi, V[:, :t_sel])


@pytest.mark.parametrize("n,r_kv,D,H,Hkv,kstd", [(2048, 0.3, 64, 8, 2, 0.02), (8192, 0.5, 128, 32, 8, 1.0),
                                                  (40000, 0.3, 64, 8, 2, 1.0), (131072, 0.3, 128, 32, 8, 1.0)])
def test_kv_select_valid_under_plain_scores(n, r_kv, D, H, Hkv, kstd):
    """The oracle's selection (scores in the documented float32 order) is a
    valid top-k of the plain float64 bound sum_j sum_d max(q kmax, q kmin),
    up to swaps within the float32 rounding band; a selection that swaps
    one kept block for a clearly lower-scored one fails the same check."""
    import kv_validity as kvv
    rng = np.random.default_rng(n)
    window = 1024 if D == 128 else 128
    q = gen.to_bf16_bits((rng.standard_normal((H, D)) * 1.3).astype(np.float32))
    nb = (n + 15) // 16
    summ = np.zeros((Hkv, nb, D, 2), np.uint16)
    for g in range(Hkv):
        keys = gen.to_bf16_bits((rng.standard_normal((n, D)) * kstd).astype(np.float32))
        summ[g] = oracle.kv_summary(keys, n)
    bud = oracle.kv_budget(n, r_kv, 4, window)
    idx, s32 = oracle.kv_select(q, summ, n, H, Hkv, r_kv, 4, window, want_scores=True)
    s64, band = kvv.plain_scores(q, summ, bud["n_cand"], bud["b_lo"])
    # the float32 scores lie within their bands of the plain ones
    assert np.all(np.abs(s32.astype(np.float64) - s64) <= band)
    for g in range(Hkv):
        kept = kvv.kept_blocks(idx[g], bud["sinks"], bud["window"], n, bud["b_lo"], bud["n_cand"])
        ok, margin = kvv.is_valid_topk(s64[g], band[g], kept, bud["k_blk"])
        assert ok, (g, margin)
        # negative control: drop the best kept block for the worst dropped one
        dropped = np.setdiff1d(np.arange(bud["n_cand"]), kept)
        bad = kept.copy()
        bad[np.argmax(s64[g][kept])] = dropped[np.argmin(s64[g][dropped])]
        assert not kvv.is_valid_topk(s64[g], band[g], bad, bud["k_blk"])[0]
