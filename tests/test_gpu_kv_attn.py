"""GPU parity of the KV summaries and the attention-scored KV selection
(bit-exact scores and index lists) and of split-K attention (partials and
merged output within 2e-3 + 1e-2|ref|) against the CPU oracle, through the
C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
from activation_kv_cache_amd import inputs as gen

from gpu_util import assert_close, assert_close_bf16, dev, host, host_u16, workspace

pytestmark = pytest.mark.gpu


def _bc():
    from activation_kv_cache_amd import binding as bc
    return bc


def _summary_host(K, n, n_cap):
    Hkv, _, D = K.shape
    s = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
    for g in range(Hkv):
        t = oracle.kv_summary(K[g], n)
        s[g, :t.shape[0]] = t
    return s


@pytest.mark.parametrize("Hkv,n_cap,n,D", [(2, 2048, 2048, 64), (2, 2048, 1999, 64), (8, 8192, 8192, 128),
                                            (8, 4096, 17, 128)])
def test_build_summary_bit_exact(Hkv, n_cap, n, D):
    bc = _bc()
    K = gen.normal_bf16(1, f"sumk{n}", (Hkv, n_cap, D), 1.0)
    s = torch.zeros((Hkv, n_cap // 16, D, 2), dtype=torch.int16, device="cuda")
    bc.bc_build_kv_summary(dev(K), n, s)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(s), _summary_host(K, n, n_cap))


KV_CASES = [
    # (name, dims, n_cap, n, r_kv, sinks, window)
    ("tiny-0.3", gen.TINY, 2048, 2048, 0.3, 4, 128),
    ("tiny-ragged", gen.TINY, 2048, 1999, 0.4, 4, 100),
    ("tiny-streaming", gen.TINY, 2048, 2048, 0.3, 4, 1024),
    ("8b-2k-0.3", gen.LLAMA8B, 2048, 2048, 0.3, 4, 1024),
    ("8b-8k-0.5", gen.LLAMA8B, 8192, 8192, 0.5, 4, 1024),
    ("8b-32k-0.3", gen.LLAMA8B, 32768, 32768, 0.3, 4, 1024),
    ("8b-128k-0.3", gen.LLAMA8B, 131072, 131072, 0.3, 4, 1024),
    ("8b-128k-0.5", gen.LLAMA8B, 131072, 131072, 0.5, 4, 1024),
    # past 8192 candidates: 16 staged keys per selecting thread, then (past
    # 16384) 32 keys read per thread
    ("tiny-160k-16-keys", gen.TINY, 160000, 160000, 0.3, 4, 128),
    ("8b-192k-16-keys", gen.LLAMA8B, 196608, 196608, 0.3, 4, 1024),
    ("tiny-320k-32-keys", gen.TINY, 320000, 320000, 0.5, 4, 128),
    # the other GQA group sizes: 1, 2 and 8 query heads per KV head
    ("g1-d64-0.3", dict(n_heads=2, n_kv_heads=2, head_dim=64), 4096, 4000, 0.3, 4, 128),
    ("g2-d128-0.3", dict(n_heads=8, n_kv_heads=4, head_dim=128), 4096, 4096, 0.3, 4, 1024),
    ("g8-d64-0.5", dict(n_heads=16, n_kv_heads=2, head_dim=64), 8192, 8192, 0.5, 4, 128),
    # the KV-window baseline: a window as long as the context leaves no
    # scored blocks, so the list is the sinks and the most recent tokens
    ("tiny-window-0.5", gen.TINY, 2048, 2000, 0.5, 4, 2000),
    ("8b-128k-window-0.3", gen.LLAMA8B, 131072, 131072, 0.3, 4, 131072),
]


@pytest.mark.parametrize("name,dims,n_cap,n,r_kv,sinks,window", KV_CASES, ids=[c[0] for c in KV_CASES])
def test_kv_score_select_bit_exact(name, dims, n_cap, n, r_kv, sinks, window):
    bc = _bc()
    H, Hkv, D = dims["n_heads"], dims["n_kv_heads"], dims["head_dim"]
    q = gen.normal_bf16(2, f"kq{name}", (H, D))
    nb = (n + 15) // 16
    # summaries straight from the seeded generator: min <= max per dim
    a = gen.normal_bf16(2, f"ka{name}", (Hkv, nb, D), 1.0)
    b = gen.normal_bf16(2, f"kb{name}", (Hkv, nb, D), 1.0)
    av, bv = oracle.bf16_to_f64(a), oracle.bf16_to_f64(b)
    summ = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
    summ[:, :nb, :, 0] = np.where(av <= bv, a, b)
    summ[:, :nb, :, 1] = np.where(av <= bv, b, a)
    pol = bc.policy(r_kv, sinks, window)
    bud = bc.bc_kv_budget(n, pol)
    ref_bud = oracle.kv_budget(n, r_kv, sinks, window)
    assert (bud["t_sel"], bud["k_blk"], bud["n_cand"]) == (ref_bud["T_sel"], ref_bud["k_blk"], ref_bud["n_cand"])
    idx = torch.full((Hkv, bud["t_sel"]), -1, dtype=torch.int32, device="cuda")
    scores = torch.empty((Hkv, max(bud["n_cand"], 1)), dtype=torch.float32, device="cuda")
    bc.bc_kv_score_select(dev(q), dev(summ), n, H, Hkv, D, pol, idx, scores)
    torch.cuda.synchronize()
    ref_idx, ref_scores = oracle.kv_select(q, summ, n, H, Hkv, r_kv, sinks, window, want_scores=True)
    if bud["n_cand"] > 0 and bud["k_blk"] > 0:
        assert np.array_equal(host(scores)[:, :bud["n_cand"]].view(np.uint32), ref_scores.view(np.uint32)), \
            "scores differ in bits"
    assert np.array_equal(host(idx), ref_idx)


def test_kv_select_ties_and_planted_block():
    """Equal scores (identical summaries) are taken lowest block first; a
    planted block aligned with the queries is always kept."""
    bc = _bc()
    dims = gen.LLAMA8B
    H, Hkv, D, n, n_cap = 32, 8, 128, 8192, 8192
    q = gen.normal_bf16(3, "tieq", (H, D))
    row = gen.normal_bf16(3, "tierow", (D,))
    summ = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
    summ[:, :, :, 0] = row
    summ[:, :, :, 1] = row
    planted = 300
    qv = oracle.bf16_to_f64(q)
    for g in range(Hkv):
        direction = np.sign(qv[4 * g:4 * g + 4].sum(0))
        summ[g, planted, :, 0] = oracle.f64_to_bf16(direction * 4.0)
        summ[g, planted, :, 1] = oracle.f64_to_bf16(direction * 4.0)
    pol = bc.policy(0.2, 4, 1024)
    bud = bc.bc_kv_budget(n, pol)
    idx = torch.full((Hkv, bud["t_sel"]), -1, dtype=torch.int32, device="cuda")
    ws = workspace(bc.bc_kv_score_select_workspace_bytes(n, Hkv, pol))
    bc.bc_kv_score_select(dev(q), dev(summ), n, H, Hkv, D, pol, idx, None, ws)
    torch.cuda.synchronize()
    got = host(idx)
    assert np.array_equal(got, oracle.kv_select(q, summ, n, H, Hkv, 0.2, 4, 1024))
    for g in range(Hkv):
        assert set(range(16 * planted, 16 * planted + 16)) <= set(got[g].tolist())


def _attn_inputs(name, dims, n_cap, std_k=1.0, std_v=1.0, planted=False):
    H, Hkv, D = dims["n_heads"], dims["n_kv_heads"], dims["head_dim"]
    q = gen.normal_bf16(4, f"aq{name}", (H, D))
    K = gen.normal_bf16(4, f"ak{name}", (Hkv, n_cap, D), std_k)
    V = gen.normal_bf16(4, f"av{name}", (Hkv, n_cap, D), std_v)
    if planted:
        # a few keys aligned with the query group give O(1) attention outputs
        qv = oracle.bf16_to_f64(q)
        rng = gen.rng(4, f"plant{name}")
        for g in range(Hkv):
            dirn = qv[g * (H // Hkv):(g + 1) * (H // Hkv)].sum(0)
            dirn = dirn / np.linalg.norm(dirn) * 3.0 * math.sqrt(D) / 4
            for t in rng.choice(n_cap, 8, replace=False):
                K[g, t] = oracle.f64_to_bf16(dirn)
    return q, K, V


ATTN_CASES = [
    # (name, dims, n_cap, n_sel, r_kv, n_splits, planted)
    ("tiny-dense", gen.TINY, 2048, 2048, 1.0, 8, False),
    ("tiny-dense-planted", gen.TINY, 2048, 2048, 1.0, 8, True),
    ("tiny-sel", gen.TINY, 2048, 2048, 0.3, 8, True),
    ("tiny-ragged-splits", gen.TINY, 2048, 1001, 1.0, 7, True),
    ("tiny-one-split", gen.TINY, 2048, 333, 1.0, 1, True),
    ("tiny-more-splits-than-rows", gen.TINY, 64, 5, 1.0, 16, False),
    ("8b-2k-dense", gen.LLAMA8B, 2048, 2048, 1.0, 32, True),
    ("8b-8k-sel", gen.LLAMA8B, 8192, 8192, 0.5, 0, True),
    ("8b-32k-dense", gen.LLAMA8B, 32768, 32768, 1.0, 0, True),
    ("8b-128k-dense", gen.LLAMA8B, 131072, 131072, 1.0, 0, True),
    ("8b-128k-sel", gen.LLAMA8B, 131072, 131072, 0.3, 0, True),
    # the other GQA group sizes the kernel is built for (1, 2 and 8 query
    # heads per KV head), dense and through an index list
    ("g1-d64-dense", dict(n_heads=4, n_kv_heads=4, head_dim=64), 1024, 1000, 1.0, 8, True),
    ("g2-d128-sel", dict(n_heads=8, n_kv_heads=4, head_dim=128), 4096, 4096, 0.3, 0, True),
    ("g8-d128-dense", dict(n_heads=16, n_kv_heads=2, head_dim=128), 2048, 2048, 1.0, 0, True),
    ("g8-d64-sel", dict(n_heads=16, n_kv_heads=2, head_dim=64), 2048, 2048, 0.3, 8, True),
    # more splits than the reduce kernel preloads (32): its looping path
    ("tiny-33-splits", gen.TINY, 2048, 2048, 1.0, 33, False),
    ("8b-2k-64-splits", gen.LLAMA8B, 2048, 2048, 1.0, 64, True),
]


@pytest.mark.parametrize("name,dims,n_cap,n,r_kv,S,planted", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_splitk_attention_vs_oracle(name, dims, n_cap, n, r_kv, S, planted):
    bc = _bc()
    H, Hkv, D = dims["n_heads"], dims["n_kv_heads"], dims["head_dim"]
    q, K, V = _attn_inputs(name, dims, n_cap, planted=planted)
    if r_kv < 1:
        summ = _summary_host(K, n, n_cap)
        lst = oracle.kv_select(q, summ, n, H, Hkv, r_kv, 4, 1024 if D == 128 else 128)
        n_sel = lst.shape[1]
    else:
        lst, n_sel = None, n
    if S == 0:
        S = bc.bc_attn_default_splits(n_sel, Hkv)
    m = torch.empty((H, S), dtype=torch.float32, device="cuda")
    l = torch.empty((H, S), dtype=torch.float32, device="cuda")
    o = torch.empty((H, S, D), dtype=torch.float32, device="cuda")
    out = torch.empty((H, D), dtype=torch.int16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    bc.bc_splitk_attn_partial(dev(q), dev(K), dev(V), None if lst is None else dev(lst), n_sel, H, Hkv, S, scale,
                              m, l, o)
    bc.bc_splitk_reduce(m, l, o, out)
    torch.cuda.synchronize()
    rm, rl, ro = oracle.attn_partial(q, K, V, lst, n_sel, H, Hkv, S, scale)
    ref64, _ = oracle.attn_reduce(rm, rl, ro)
    gm, gl, go = host(m), host(l), host(o)
    empty = np.isneginf(rm)
    assert np.array_equal(np.isneginf(gm), empty)
    assert np.all(gl[empty] == 0) and np.all(go[empty] == 0)
    ne = ~empty
    assert_close(gm[ne], rm[ne], "m", atol=1e-4, rtol=1e-5)
    # the kernel rounds each softmax weight to bf16 before adding it into both
    # l and o (bf16 x bf16 pairs into fp32 on v_dot2), so l carries a relative
    # error up to 2^-8 against the exact sum
    assert_close(gl[ne], rl[ne], "l", atol=1e-5, rtol=2.0 ** -8)
    assert_close((go / np.where(gl > 0, gl, 1)[..., None])[ne], (ro / np.where(rl > 0, rl, 1)[..., None])[ne], "o/l")
    rel = assert_close_bf16(host_u16(out), ref64, name)
    assert rel < 1e-2, f"rel-L2 {rel}"


@pytest.mark.parametrize("H,S,D", [(8, 1, 64), (8, 2, 128), (32, 16, 128), (32, 31, 64), (32, 32, 128),
                                   (32, 33, 128), (8, 64, 64), (4, 257, 128)])
def test_splitk_reduce_vs_oracle(H, S, D):
    """bc_splitk_reduce alone on seeded partials (some splits empty: m = -inf,
    l = o = 0; one head with every split empty) against the oracle's merge,
    on both sides of the 32 splits the kernel preloads."""
    bc = _bc()
    rng = gen.rng(0, f"reduce/{H}/{S}/{D}")
    m = rng.normal(0.0, 2.0, size=(H, S)).astype(np.float32)
    l = rng.uniform(0.5, 5.0, size=(H, S)).astype(np.float32)
    o = (rng.standard_normal(size=(H, S, D)) * l[..., None]).astype(np.float32)
    empty = rng.random(size=(H, S)) < 0.2
    empty[H - 1, :] = True
    m[empty] = -np.inf
    l[empty] = 0.0
    o[empty] = 0.0
    out = torch.empty((H, D), dtype=torch.int16, device="cuda")
    bc.bc_splitk_reduce(torch.from_numpy(m).cuda(), torch.from_numpy(l).cuda(), torch.from_numpy(o).cuda(), out)
    torch.cuda.synchronize()
    ref64, _ = oracle.attn_reduce(m, l, o)
    got = host_u16(out)
    assert np.all(got[H - 1] == 0)
    assert_close_bf16(got, ref64, f"reduce H={H} S={S} D={D}")


def test_dense_attention_equals_identity_list():
    """idx = NULL and idx = 0..n-1 read the same rows through the same kernel: bit-identical."""
    bc = _bc()
    dims = gen.LLAMA8B
    H, Hkv, D, n = 32, 8, 128, 4096
    q, K, V = _attn_inputs("ident", dims, n)
    S = bc.bc_attn_default_splits(n, Hkv)
    outs = []
    for lst in (None, np.tile(np.arange(n, dtype=np.int32), (Hkv, 1))):
        m = torch.empty((H, S), dtype=torch.float32, device="cuda")
        l = torch.empty_like(m)
        o = torch.empty((H, S, D), dtype=torch.float32, device="cuda")
        out = torch.empty((H, D), dtype=torch.int16, device="cuda")
        bc.bc_splitk_attn_partial(dev(q), dev(K), dev(V), None if lst is None else dev(lst), n, H, Hkv, S,
                                  1 / math.sqrt(D), m, l, o)
        bc.bc_splitk_reduce(m, l, o, out)
        outs.append((m, l, o, out))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.gpu
@pytest.mark.parametrize("name,dims,n_cap,n,r_kv", [("tiny", gen.TINY, 2048, 2000, 0.3),
                                                    ("8b-8k", gen.LLAMA8B, 8192, 8192, 0.5)])
def test_kv_compact_and_sel_mode_attention(name, dims, n_cap, n, r_kv):
    """bc_kv_compact (the sel mode's gather) is bit-exact against the oracle's
    gather, and the dense kernel over the compacted cache gives the same bits
    as the index-list kernel over the original cache, and the oracle's
    attention over the list within tolerance."""
    bc = _bc()
    H, Hkv, D = dims["n_heads"], dims["n_kv_heads"], dims["head_dim"]
    window = 128 if dims is gen.TINY else 1024
    q, K, V = _attn_inputs(f"kc{name}", dims, n_cap)
    summ = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
    for g in range(Hkv):
        t = oracle.kv_summary(K[g], n)
        summ[g, :t.shape[0]] = t
    lst = oracle.kv_select(q, summ, n, H, Hkv, r_kv, 4, window)
    t_sel = lst.shape[1]
    n_out = t_sel + 16
    Kc = torch.zeros((Hkv, n_out, D), dtype=torch.int16, device="cuda")
    Vc = torch.zeros_like(Kc)
    bc.bc_kv_compact(dev(K), dev(V), dev(lst), t_sel, Kc, Vc)
    Kr, Vr = oracle.kv_compact(K, V, lst, n_out)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(Kc), Kr) and np.array_equal(host_u16(Vc), Vr)
    S = bc.bc_attn_default_splits(t_sel, Hkv)
    outs = []
    for kk, vv, idx in ((Kc, Vc, None), (dev(K), dev(V), dev(lst))):
        m = torch.empty((H, S), dtype=torch.float32, device="cuda")
        l = torch.empty_like(m)
        o = torch.empty((H, S, D), dtype=torch.float32, device="cuda")
        out = torch.empty((H, D), dtype=torch.int16, device="cuda")
        bc.bc_splitk_attn_partial(dev(q), kk, vv, idx, t_sel, H, Hkv, S, 1 / math.sqrt(D), m, l, o)
        bc.bc_splitk_reduce(m, l, o, out)
        outs.append((m, l, o, out))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    ref64, _ = oracle.attn_reduce(*oracle.attn_partial(q, K, V, lst, t_sel, H, Hkv, S))
    assert_close_bf16(host_u16(outs[0][3]), ref64)


def test_stream_read_probe_checksum():
    """The read probe (a measurement helper) reads every 16-byte piece of its
    source: its per-work-group checksums match a host replay of the lane
    assignment (work-group g streams share g; lane t of wave 0 takes pieces
    t, t + 2048, ... and each one's partner 1024 pieces on)."""
    bc = _bc()
    nbytes = 8 << 20
    words = np.arange(nbytes // 4, dtype=np.uint32) * np.uint32(2654435761)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((256,), -1, dtype=torch.int32, device="cuda")
    bc.bc_stream_read(src, sink)
    torch.cuda.synchronize()
    got = host(sink).view(np.uint32)
    quads = words.reshape(256, -1, 4)
    x4 = quads[..., 0] ^ quads[..., 1] ^ quads[..., 2] ^ quads[..., 3]   # [group][piece]
    n16 = x4.shape[1]
    ref = np.zeros(256, np.uint64)
    for t in range(64):
        acc = np.zeros(256, np.uint32)
        for i in range(t, n16, 2048):
            acc ^= x4[:, i]
            if i + 1024 < n16:
                acc ^= x4[:, i + 1024]
        ref += acc
    assert np.array_equal(got, (ref % (1 << 32)).astype(np.uint32))



@pytest.mark.parametrize("n,r_kv", [(2048, 0.7), (32768, 0.3), (32768, 0.5), (131072, 0.3), (131072, 0.5)],
                         ids=["8b-2k-0.7", "8b-32k-0.3", "8b-32k-0.5", "8b-128k-0.3", "8b-128k-0.5"])
def test_kv_selection_valid_under_plain_scores(n, r_kv):
    """Order-independent check at Llama-3.1-8B dims: the GPU's kept blocks
    form a valid top-k of the plain float64 bound sum_j sum_d max(q kmax,
    q kmin) (numpy, no oracle code), up to swaps within the float32 rounding
    band of each score; the GPU's float32 scores lie within those bands."""
    import kv_validity as kvv
    bc = _bc()
    H, Hkv, D = 32, 8, 128
    kc = gen.device_normal_bf16(51, f"validk{n}", (Hkv, n, D), 1.0)
    summ = torch.zeros((Hkv, n // 16, D, 2), dtype=torch.int16, device="cuda")
    bc.bc_build_kv_summary(kc, n, summ)
    q = gen.device_normal_bf16(51, f"validq{n}", (H, D), 1.3)
    pol = bc.policy(r_kv, 4, 1024)
    bud = bc.bc_kv_budget(n, pol)
    assert bud["k_blk"] > 0
    idx = torch.full((Hkv, bud["t_sel"]), -1, dtype=torch.int32, device="cuda")
    scores = torch.empty((Hkv, bud["n_cand"]), dtype=torch.float32, device="cuda")
    ws = workspace(bc.bc_kv_score_select_workspace_bytes(n, Hkv, pol))
    print(f"[kv-valid] n={n} r_kv={r_kv} k_blk={bud['k_blk']} n_cand={bud['n_cand']}", flush=True)
    bc.bc_kv_score_select(q, summ, n, H, Hkv, D, pol, idx, scores, ws)
    torch.cuda.synchronize()
    s64, band = kvv.plain_scores(host_u16(q), host_u16(summ), bud["n_cand"], bud["b_lo"])
    s32 = host(scores).astype(np.float64)
    assert np.all(np.abs(s32 - s64) <= band), "float32 scores outside their rounding bands"
    ids = host(idx)
    margins = []
    for g in range(Hkv):
        kept = kvv.kept_blocks(ids[g], bud["sinks"], bud["window"], n, bud["b_lo"], bud["n_cand"])
        ok, margin = kvv.is_valid_topk(s64[g], band[g], kept, bud["k_blk"])
        margins.append(margin)
        assert ok, f"head {g}: not a top-{bud['k_blk']} of the plain scores (margin {margin:.3g})"
    print(f"[kv-valid] margins (>= 0: valid) min {min(margins):.3g}", flush=True)
