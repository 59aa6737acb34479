"""GPU parity of the whole decoder layer (bc_decode_layer) and the LM head
against the CPU oracle.

Stage by stage with teacher forcing: the oracle recomputes every stage from
the GPU's own inputs to that stage (taps), so selections are compared bit for
bit and floating-point stages within 2e-3 + 1e-2|ref|.  With both keeps at 1
the layer is also compared end to end without forcing."""
import functools

import numpy as np
import pytest
import torch

import oracle
from activation_kv_cache_amd import inputs as gen

from gpu_util import assert_close, assert_close_bf16, dev, host, host_u16, workspace

pytestmark = pytest.mark.gpu

FP_STAGES = ("x1", "q", "k", "v", "a", "h_mid", "x2", "hff", "h_out")
# a mid-size shape whose o GEMV chunks (64 channels) split its 128-wide heads
MID = dict(d=1024, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=2816, vocab=1000, n_layers=1)
IDX_STAGES = ("idx_qkv", "idx_kv", "idx_o", "idx_gu", "idx_down")


def _bc():
    from activation_kv_cache_amd import binding as bc
    return bc


@functools.lru_cache(maxsize=1)
def _layer_inputs(seed, dims_items, n_cap, k_std):
    """Weights and cache of one layer (the full-size cases share them; they
    take most of such a case's time to draw)."""
    dims = dict(dims_items)
    return gen.layer_weights(seed, dims), gen.kv_cache(seed, dims, n_cap, k_std)


def _run_layer(dims, n_cap, n, r_p, r_kv, sinks, window, n_splits, seed, k_std=0.02, plant=False):
    bc = _bc()
    H, Hkv, D, d, dff = dims["n_heads"], dims["n_kv_heads"], dims["head_dim"], dims["d"], dims["d_ff"]
    W, (K, V) = _layer_inputs(seed, tuple(sorted(dims.items())), n_cap, k_std)
    h = gen.activation_bf16(seed, "h0", d)
    summ = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
    for g in range(Hkv):
        s = oracle.kv_summary(K[g], n - 1)
        summ[g, :s.shape[0]] = s
    w = {k: dev(v) for k, v in W.items()}
    w_gu = torch.empty(2 * d * dff, dtype=torch.int16, device="cuda")
    bc.bc_pack_gate_up(w["gate"], w["up"], w_gu)
    kc, vc, sm, hh = dev(K), dev(V), dev(summ), dev(h)
    md = bc.dims(dims)
    pol = bc.policy(r_kv, sinks, window)
    bud = bc.bc_kv_budget(n, pol)
    n_sel = bud["t_sel"]
    S = n_splits or bc.bc_attn_default_splits(n_sel, Hkv)
    ws = workspace(bc.bc_layer_workspace_bytes(md, n_cap, S))
    k_d, k_ff = oracle.channel_keep(r_p, d), oracle.channel_keep(r_p, dff)
    i16, i32 = torch.int16, torch.int32
    sizes = {"x1": (d, i16), "idx_qkv": (k_d, i32), "q": (H * D, i16), "k": (Hkv * D, i16), "v": (Hkv * D, i16),
             "idx_kv": (Hkv * n_sel, i32), "a": (H * D, i16), "idx_o": (k_d, i32), "h_mid": (d, i16),
             "x2": (d, i16), "idx_gu": (k_d, i32), "hff": (dff, i16), "idx_down": (k_ff, i32),
             "attn_m": (H * S, torch.float32), "attn_l": (H * S, torch.float32), "attn_o": (H * S * D, torch.float32)}
    taps = {k: torch.full((n,), -1, dtype=t, device="cuda") for k, (n, t) in sizes.items()}
    layer = bc.make_layer(bc.packed_tiles(w["qkv"]), bc.packed_tiles(w["o"]), w_gu, bc.packed_tiles(w["down"]),
                          w["g1"], w["g2"], kc, vc, sm)
    step = bc.make_step(n, r_p, pol, S, taps=bc.make_taps(**taps))
    bc.bc_decode_layer(md, layer, step, hh, ws)
    torch.cuda.synchronize()
    got = {}
    for k, t in taps.items():
        got[k] = host_u16(t) if t.dtype == torch.int16 else host(t)
    got["h_out"] = host_u16(hh)
    got["K"], got["V"], got["summ"] = host_u16(kc), host_u16(vc), host_u16(sm)
    return W, K, V, h, summ, got, S


def _shape_forced(got, dims, r_p, r_kv):
    H, Hkv, D = dims["n_heads"], dims["n_kv_heads"], dims["head_dim"]
    f = {k: got[k] for k in ("x1", "a", "h_mid", "x2", "hff")}
    f["q"] = got["q"].reshape(H, D)
    f["k"] = got["k"].reshape(Hkv, D)
    f["v"] = got["v"].reshape(Hkv, D)
    if r_p < 1:
        for k in ("idx_qkv", "idx_o", "idx_gu", "idx_down"):
            f[k] = got[k]
    if r_kv < 1:
        f["idx_kv"] = got["idx_kv"].reshape(Hkv, -1)
    return f


LAYER_CASES = [
    # (name, dims, n_cap, n, r_p, r_kv, sinks, window, n_splits)
    ("tiny-dense", gen.TINY, 2048, 2048, 1.0, 1.0, 4, 128, 8),
    ("tiny-proj", gen.TINY, 2048, 2048, 0.5, 1.0, 4, 128, 8),
    ("tiny-kv", gen.TINY, 2048, 2048, 1.0, 0.3, 4, 128, 8),
    ("tiny-both", gen.TINY, 2048, 2048, 0.5, 0.3, 4, 128, 8),
    ("tiny-ragged-ctx", gen.TINY, 2064, 2051, 0.7, 0.3, 4, 128, 5),
    ("tiny-first-token", gen.TINY, 64, 1, 0.5, 1.0, 4, 128, 1),
    # dense list, few tokens: the current token (attended from LDS by the
    # work-group that appends it) carries a large share of the weights; the
    # last split holds only that token in the second case
    ("tiny-short-ctx", gen.TINY, 64, 17, 1.0, 1.0, 4, 128, 3),
    ("tiny-split-of-one", gen.TINY, 64, 13, 1.0, 1.0, 4, 128, 4),
    # more attention splits than the o GEMV prologue combines: a reduce
    # kernel forms the attention output
    ("tiny-dense-40-splits", gen.TINY, 2048, 2048, 1.0, 1.0, 4, 128, 40),
    ("tiny-first-token-dense", gen.TINY, 64, 1, 1.0, 1.0, 4, 128, 1),
    # head_dim 128 over 64-channel o-GEMV chunks: a chunk holds half a head
    ("mid-half-head-chunks", MID, 1024, 1000, 1.0, 1.0, 4, 128, 4),
    # over 2048 candidate blocks: a selection kernel ranks the kept blocks
    # once per KV head and the attention work-groups copy their ranks
    ("tiny-long-ctx-ranked", gen.TINY, 40960, 40000, 0.7, 0.3, 4, 128, 0),
    ("8b-2k-dense", gen.LLAMA8B, 2048, 2048, 1.0, 1.0, 4, 1024, 0),
    ("8b-2k-both-0.5-0.3", gen.LLAMA8B, 2048, 2048, 0.5, 0.3, 4, 1024, 0),
    ("8b-8k-both-0.7-0.3", gen.LLAMA8B, 8192, 8192, 0.7, 0.3, 4, 1024, 0),
    # the headline and composed steps' own layer: 131072 tokens, the default
    # 32 splits (the o GEMV merges them when dense; the kept blocks are
    # ranked by their own kernel when sparse)
    ("8b-128k-dense", gen.LLAMA8B, 131072, 131072, 1.0, 1.0, 4, 1024, 0),
    ("8b-128k-both-0.5-0.3", gen.LLAMA8B, 131072, 131072, 0.5, 0.3, 4, 1024, 0),
    # over 8192 candidate blocks at 8 KV heads: the scoring work-groups take
    # more than 256 blocks each (their last loads issued after q is formed)
    # and the ranking kernel holds 16 keys per thread
    ("8b-160k-kv-0.3", gen.LLAMA8B, 163840, 163840, 1.0, 0.3, 4, 1024, 0),
    # the KV-window baseline (sinks and the most recent tokens, no scoring)
    # through the same attention kernel
    ("tiny-kv-window", gen.TINY, 2048, 2048, 1.0, 0.3, 4, 2048, 8),
    ("8b-128k-kv-window-0.3", gen.LLAMA8B, 131072, 131072, 1.0, 0.3, 4, 131072, 0),
    # GQA group sizes 1 and 8 through the whole layer
    ("tiny-g1-both", dict(gen.TINY, n_kv_heads=8), 2048, 2048, 0.5, 0.3, 4, 128, 8),
    ("tiny-g8-dense", dict(gen.TINY, n_kv_heads=1), 2048, 2048, 1.0, 1.0, 4, 128, 8),
    ("tiny-g8-both", dict(gen.TINY, n_kv_heads=1), 2048, 2048, 0.5, 0.3, 4, 128, 8),
]


@pytest.mark.parametrize("name,dims,n_cap,n,r_p,r_kv,sinks,window,S", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_decode_layer_teacher_forced(name, dims, n_cap, n, r_p, r_kv, sinks, window, S):
    W, K, V, h, summ, got, S = _run_layer(dims, n_cap, n, r_p, r_kv, sinks, window, S, seed=9)
    forced = _shape_forced(got, dims, r_p, r_kv)
    Ko, Vo, so = K.copy(), V.copy(), summ.copy()
    ref = oracle.decode_layer(h, W, Ko, Vo, so, n, dims, r_p, r_kv, sinks, window, S, forced=forced)
    for st in IDX_STAGES:
        if ref.get(st) is None:
            continue
        assert np.array_equal(got[st].reshape(ref[st].shape), ref[st]), f"{name}: {st} differs"
    for st in FP_STAGES:
        r = ref[st]
        assert_close_bf16(got[st], oracle.bf16_to_f64(r), f"{name}: {st}")
    # the cache holds the GPU's new row and the refreshed summary matches the oracle's
    assert np.array_equal(got["K"][:, n - 1], forced["k"]) and np.array_equal(got["V"][:, n - 1], forced["v"])
    assert np.array_equal(got["summ"], so)


@pytest.mark.parametrize("dims,n_cap,n,S,r_kv", [(gen.TINY, 2048, 2048, 8, 1.0), (gen.TINY, 64, 1, 1, 1.0),
                                                (gen.TINY, 2048, 2048, 32, 1.0), (gen.TINY, 2048, 2048, 40, 1.0),
                                                (gen.TINY, 2048, 2048, 8, 0.3), (MID, 1024, 1000, 4, 1.0),
                                                (gen.LLAMA8B, 2048, 2048, 0, 1.0)],
                         ids=["tiny-8-splits", "tiny-first-token", "tiny-32-splits", "tiny-40-splits-reduce-kernel",
                              "tiny-kv-0.3", "mid-half-head-chunks", "8b-2k"])
def test_attention_output_equals_reduce_of_partials(dims, n_cap, n, S, r_kv):
    """The layer's attention output equals, bit for bit, bc_splitk_reduce
    over the layer's own split partials: a dense o GEMV forms it in its
    prologue (up to 32 splits, no reduce launch), otherwise the reduce kernel
    does; both follow one combine order."""
    bc = _bc()
    W, K, V, h, summ, got, S = _run_layer(dims, n_cap, n, 1.0, r_kv, 4, 128, S, seed=5)
    H, D = dims["n_heads"], dims["head_dim"]
    m = dev(got["attn_m"].reshape(H, S))
    l = dev(got["attn_l"].reshape(H, S))
    o = dev(got["attn_o"].reshape(H, S, D))
    out = torch.full((H * D,), -1, dtype=torch.int16, device="cuda")
    bc.bc_splitk_reduce(m, l, o, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), got["a"])


def _bf16_ulp(x):
    """One unit in the last place of bf16 values of magnitude |x| (8
    significant bits: 2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return 2.0 ** (np.maximum(e, -126) - 7)


@pytest.mark.parametrize("dims,n_cap,n", [(gen.TINY, 2048, 2048), (gen.LLAMA8B, 2048, 2048)], ids=["tiny", "8b-2k"])
def test_dense_layer_end_to_end(dims, n_cap, n):
    """Without teacher forcing the GPU and the oracle round their stored bf16
    intermediates independently, so a stored value may differ by one bf16
    ulp (the stage tests above bound each stage given its inputs).  Two such
    differences reach h_out: one ulp of the residual h_mid, and one ulp of
    each SwiGLU output f_i carried through W_down.  The elementwise bound adds
    ulp(h_mid_o) and 4 standard deviations of that propagated noise,
    4 * sqrt(sum_i (W_down[i, o] * ulp(f_i))^2), to 2e-3 + 1e-2|ref|; the
    relative L2 error of the whole vector must stay below 1e-2."""
    W, K, V, h, summ, got, S = _run_layer(dims, n_cap, n, 1.0, 1.0, 4, 1024, 0, seed=10)
    ref = oracle.decode_layer(h, W, K.copy(), V.copy(), summ.copy(), n, dims, 1.0, 1.0, 4, 1024, S)
    g = oracle.bf16_to_f64(got["h_out"]).reshape(-1)
    r = oracle.bf16_to_f64(ref["h_out"]).reshape(-1)
    wd = oracle.bf16_to_f64(W["down"]).astype(np.float32)
    uf = _bf16_ulp(oracle.bf16_to_f64(ref["hff"])).astype(np.float32).reshape(-1)
    noise = np.sqrt((wd * wd).T.astype(np.float64) @ (uf.astype(np.float64) ** 2))
    tol = 2e-3 + 1e-2 * np.abs(r) + _bf16_ulp(oracle.bf16_to_f64(ref["h_mid"])).reshape(-1) + 4 * noise
    err = np.abs(g - r)
    rel = np.linalg.norm(g - r) / np.linalg.norm(r)
    assert (err <= tol).all(), f"h_out: {(err > tol).sum()} of {err.size} outside; max err {err.max():.3g}"
    assert rel < 1e-2, f"h_out: rel-L2 {rel:.3g}"


def test_lm_head_tiny():
    bc = _bc()
    dims = dict(gen.TINY, vocab=1000)
    d, V = dims["d"], dims["vocab"]
    h = gen.activation_bf16(12, "lmh", d)
    g = gen.to_bf16_bits(np.ones(d, np.float32))
    wt = gen.normal_bf16(12, "lmw", (d, V), 0.02)
    md = bc.dims(dims)
    ws = workspace(bc.bc_lm_head_workspace_bytes(md))
    logits = torch.empty(V, dtype=torch.float32, device="cuda")
    tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    bc.bc_lm_head(md, dev(h), dev(g), bc.packed_tiles(dev(wt)), logits, tok, 1e-5, ws)
    torch.cuda.synchronize()
    _, y64, arg = oracle.lm_head(h, g, wt)
    lg = host(logits)
    assert_close(lg, y64, "logits")
    assert int(host(tok)[0]) == int(np.argmax(lg))
    assert y64[int(host(tok)[0])] >= y64[arg] - 1e-2


def test_lm_head_8b_sampled():
    """Full 8B head (4096 x 128256, 1.05 GB): logits checked at sampled columns."""
    bc = _bc()
    dims = gen.LLAMA8B
    d, V = dims["d"], dims["vocab"]
    h = gen.activation_bf16(13, "lmh8", d)
    g = gen.to_bf16_bits(np.ones(d, np.float32))
    wt = gen.device_normal_bf16(13, "lmw8", (d, V), 0.02)
    md = bc.dims(dims)
    ws = workspace(bc.bc_lm_head_workspace_bytes(md))
    logits = torch.empty(V, dtype=torch.float32, device="cuda")
    tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    bc.bc_lm_head(md, dev(h), dev(g), bc.packed_tiles(wt), logits, tok, 1e-5, ws)
    torch.cuda.synchronize()
    cols = np.sort(gen.rng(13, "lmcols").choice(V, 2048, replace=False))
    sub = host_u16(wt[:, torch.from_numpy(cols).cuda()].contiguous())
    x = oracle.rmsnorm(h, g)
    y64, _ = oracle.sparse_gemv(sub, x)
    lg = host(logits)
    assert_close(lg[cols], y64, "sampled logits")
    assert int(host(tok)[0]) == int(np.argmax(lg))


def test_pack_layouts_bit_exact():
    """bc_pack_weight_tiles and bc_pack_gate_up against a numpy re-layout."""
    bc = _bc()
    d_in, d_out = 96, 328            # two full tiles and a 72-wide one
    wt = gen.normal_bf16(14, "pk", (d_in, d_out))
    got = host_u16(bc.packed_tiles(dev(wt)))
    want = []
    for t in range(0, d_out, 128):
        want.append(wt[:, t:t + 128].reshape(-1))
    assert np.array_equal(got, np.concatenate(want))
    d, dff = 40, 1408 // 8           # d_ff 176: groups of 64, 64, 48
    gate = gen.normal_bf16(14, "pkg", (d, dff))
    up = gen.normal_bf16(14, "pku", (d, dff))
    out = torch.empty(2 * d * dff, dtype=torch.int16, device="cuda")
    bc.bc_pack_gate_up(dev(gate), dev(up), out)
    inter = np.concatenate([np.concatenate([gate[:, g:g + 64], up[:, g:g + 64]], axis=1)
                            for g in range(0, dff, 64)], axis=1)
    want = [inter[:, t:t + 128].reshape(-1) for t in range(0, 2 * dff, 128)]
    assert np.array_equal(host_u16(out), np.concatenate(want))


def test_tiled_gemv_equals_plain():
    """The tile-major layout gives the same result bits as the plain one."""
    bc = _bc()
    d_in, d_out = 4096, 6144
    wt = gen.normal_bf16(15, "tg", (d_in, d_out), 0.02)
    x = gen.activation_bf16(15, "tgx", d_in)
    for r_p in (1.0, 0.5):
        k = oracle.channel_keep(r_p, d_in)
        idx = None if r_p >= 1 else dev(oracle.select_channels(x, k))
        ws = workspace(bc.bc_sparse_gemv_workspace_bytes(d_out, k))
        y1 = torch.empty(d_out, dtype=torch.int16, device="cuda")
        y2 = torch.empty(d_out, dtype=torch.int16, device="cuda")
        bc.bc_sparse_gemv(dev(wt), dev(x), idx, k, y1, ws)
        bc.bc_sparse_gemv_tiled(bc.packed_tiles(dev(wt)), d_in, d_out, dev(x), idx, k, y2, ws)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)


@pytest.mark.parametrize("r_p,r_kv", [(1.0, 1.0), (0.5, 0.3), (0.7, 1.0), (1.0, 0.3)])
def test_decode_step_equals_layer_chain(r_p, r_kv):
    """bc_decode_step (fused across layers) gives the same bits as
    bc_decode_layer per layer followed by bc_lm_head."""
    bc = _bc()
    dims = dict(gen.TINY, vocab=1000, n_layers=3)
    d, dff, Hkv, D = dims["d"], dims["d_ff"], dims["n_kv_heads"], dims["head_dim"]
    n_cap, n, S = 1024, 1000, 4
    md = bc.dims(dims)
    pol = bc.policy(r_kv, 4, 64)
    layers, caches = [], []
    for li in range(3):
        W = gen.layer_weights(20, dims, layer=li)
        w = {k: dev(v) for k, v in W.items()}
        w_gu = torch.empty(2 * d * dff, dtype=torch.int16, device="cuda")
        bc.bc_pack_gate_up(w["gate"], w["up"], w_gu)
        K, V = gen.kv_cache(20, dims, n_cap, 0.5, layer=li)
        summ = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
        for g in range(Hkv):
            t = oracle.kv_summary(K[g], n - 1)
            summ[g, :t.shape[0]] = t
        layers.append(dict(qkv=bc.packed_tiles(w["qkv"]), o=bc.packed_tiles(w["o"]), gu=w_gu,
                           down=bc.packed_tiles(w["down"]), g1=w["g1"], g2=w["g2"]))
        caches.append((K, V, summ))
    g_final = dev(gen.to_bf16_bits(np.ones(d, np.float32)))
    w_head = bc.packed_tiles(dev(gen.normal_bf16(20, "head", (d, dims["vocab"]), 0.02)))
    h0 = gen.activation_bf16(20, "h0", d)

    def fresh():
        kv = [(dev(K), dev(V), dev(sm)) for K, V, sm in caches]
        cl = [bc.make_layer(l["qkv"], l["o"], l["gu"], l["down"], l["g1"], l["g2"], *kv[i])
              for i, l in enumerate(layers)]
        return kv, cl

    st = bc.make_step(n, r_p, pol, S)
    kv1, cl1 = fresh()
    h1 = dev(h0)
    ws1 = workspace(bc.bc_layer_workspace_bytes(md, n_cap, S))
    for c in cl1:
        bc.bc_decode_layer(md, c, st, h1, ws1)
    lg1 = torch.empty(dims["vocab"], dtype=torch.float32, device="cuda")
    tk1 = torch.empty(1, dtype=torch.int32, device="cuda")
    bc.bc_lm_head(md, h1, g_final, w_head, lg1, tk1, 1e-5, workspace(bc.bc_lm_head_workspace_bytes(md)))
    kv2, cl2 = fresh()
    h2 = dev(h0)
    arr = bc.make_layer_array(cl2)
    lg2 = torch.empty_like(lg1)
    tk2 = torch.empty_like(tk1)
    bc.bc_decode_step(md, arr, g_final, w_head, st, h2, lg2, tk2, workspace(bc.bc_step_workspace_bytes(md, n_cap, S)))
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
    assert torch.equal(lg1, lg2) and torch.equal(tk1, tk2)
    for a, b in zip(kv1, kv2):
        for x, y in zip(a, b):
            assert torch.equal(x, y)
