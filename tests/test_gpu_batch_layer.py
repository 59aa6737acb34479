"""GPU parity of the batched decoder layer and step (bc_decode_layer_batch,
bc_decode_step_batch: sequences sharing the weights, the projections read
once for the union of their channel lists) against the CPU oracle, sequence
by sequence.

Each sequence's stages are teacher-forced from the GPU's own inputs to them
(taps): the channel and KV index sets bit for bit, floating-point stages
within 2e-3 + 1e-2|ref|, the cache's new row and the refreshed block summary
bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from activation_kv_cache_amd import inputs as gen

from gpu_util import assert_close, assert_close_bf16, dev, host, host_u16, workspace

pytestmark = pytest.mark.gpu

FP = ("x1", "q", "k", "v", "a", "h_mid", "x2", "hff")
IDX = ("idx_qkv", "idx_o", "idx_gu", "idx_down")


def _packed(W, dims):
    from activation_kv_cache_amd import binding as bc
    d, dff = dims["d"], dims["d_ff"]
    w = {k: dev(v) for k, v in W.items()}
    w_gu = torch.empty(2 * d * dff, dtype=torch.int16, device="cuda")
    bc.bc_pack_gate_up(w["gate"], w["up"], w_gu)
    return dict(qkv=bc.packed_tiles(w["qkv"]), o=bc.packed_tiles(w["o"]), gu=w_gu, down=bc.packed_tiles(w["down"]),
                g1=w["g1"], g2=w["g2"])


def _caches(dims, n_cap, n, seed, layer, B, k_std):
    Hkv, D = dims["n_kv_heads"], dims["head_dim"]
    out = []
    for b in range(B):
        K = gen.normal_bf16(seed, f"bl{layer}/k{b}", (Hkv, n_cap, D), k_std)
        V = gen.normal_bf16(seed, f"bl{layer}/v{b}", (Hkv, n_cap, D), 1.0)
        summ = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
        for g in range(Hkv):
            s = oracle.kv_summary(K[g], n - 1)
            summ[g, :s.shape[0]] = s
        out.append((K, V, summ))
    return out


CASES = [
    # (name, dims, B, n_cap, n, r_p, r_kv, window, S)
    ("tiny-b1-dense", gen.TINY, 1, 2048, 2000, 1.0, 1.0, 128, 8),
    ("tiny-b2-proj", gen.TINY, 2, 2048, 2000, 0.5, 1.0, 128, 8),
    ("tiny-b3-kv", gen.TINY, 3, 2048, 2000, 1.0, 0.3, 128, 8),
    ("tiny-b4-both", gen.TINY, 4, 2048, 2000, 0.5, 0.3, 128, 8),
    ("tiny-b4-both-0.7", gen.TINY, 4, 2048, 2048, 0.7, 0.5, 128, 0),
    ("8b-2k-b2-both", gen.LLAMA8B, 2, 2048, 2048, 0.5, 0.3, 1024, 0),
]


@pytest.mark.parametrize("name,dims,B,n_cap,n,r_p,r_kv,window,S", CASES, ids=[c[0] for c in CASES])
def test_batch_layer_teacher_forced(name, dims, B, n_cap, n, r_p, r_kv, window, S):
    from activation_kv_cache_amd import binding as bc
    H, Hkv, D, d, dff = dims["n_heads"], dims["n_kv_heads"], dims["head_dim"], dims["d"], dims["d_ff"]
    W = gen.layer_weights(81, dims)
    pw = _packed(W, dims)
    caches = _caches(dims, n_cap, n, 81, 0, B, 0.5)
    h = np.stack([gen.activation_bf16(81, f"bh{b}", d) for b in range(B)])
    md = bc.dims(dims)
    pol = bc.policy(r_kv, 4, window)
    bud = bc.bc_kv_budget(n, pol)
    n_sel = bud["t_sel"]
    S = S or bc.bc_attn_default_splits(n_sel, Hkv)
    dev_caches = [(dev(K), dev(V), dev(sm)) for K, V, sm in caches]
    layers = [bc.make_layer(pw["qkv"], pw["o"], pw["gu"], pw["down"], pw["g1"], pw["g2"], *c) for c in dev_caches]
    arr = bc.make_layer_array(layers)
    k_d, k_ff = oracle.channel_keep(r_p, d), oracle.channel_keep(r_p, dff)
    i16, i32 = torch.int16, torch.int32
    sizes = {"x1": (d, i16), "q": (H * D, i16), "k": (Hkv * D, i16), "v": (Hkv * D, i16), "a": (H * D, i16),
             "h_mid": (d, i16), "x2": (d, i16), "hff": (dff, i16)}
    if r_p < 1:
        sizes.update(idx_qkv=(k_d, i32), idx_o=(k_d, i32), idx_gu=(k_d, i32), idx_down=(k_ff, i32))
    if r_kv < 1:
        sizes["idx_kv"] = (Hkv * n_sel, i32)
    taps = [{k: torch.full((m,), -1, dtype=t, device="cuda") for k, (m, t) in sizes.items()} for _ in range(B)]
    tarr = bc.make_taps_array([bc.make_taps(**t) for t in taps])
    hh = dev(h)
    ws = workspace(bc.bc_layer_batch_workspace_bytes(md, B, n_cap, S))
    print(f"[batch-layer] {name}: B={B} n={n} r_p={r_p} r_kv={r_kv} S={S}", flush=True)
    bc.bc_decode_layer_batch(md, arr, bc.make_step(n, r_p, pol, S), hh, ws, taps_array=tarr)
    torch.cuda.synchronize()
    h_out = host_u16(hh)
    for b in range(B):
        got = {k: (host_u16(t) if t.dtype == torch.int16 else host(t)) for k, t in taps[b].items()}
        forced = {k: got[k] for k in ("x1", "a", "h_mid", "x2", "hff")}
        forced["q"] = got["q"].reshape(H, D)
        forced["k"] = got["k"].reshape(Hkv, D)
        forced["v"] = got["v"].reshape(Hkv, D)
        for k in IDX:
            if k in got:
                forced[k] = got[k]
        if r_kv < 1:
            forced["idx_kv"] = got["idx_kv"].reshape(Hkv, n_sel)
        K, V, summ = caches[b]
        Ko, Vo, so = K.copy(), V.copy(), summ.copy()
        ref = oracle.decode_layer(h[b], W, Ko, Vo, so, n, dims, r_p, r_kv, 4, window, S, forced=forced)
        for k in IDX + ("idx_kv",):
            if ref.get(k) is not None and k in got:
                assert np.array_equal(got[k].reshape(ref[k].shape), ref[k]), f"{name} seq {b}: {k} differs"
        for st in FP:
            assert_close_bf16(got[st], oracle.bf16_to_f64(ref[st]), f"{name} seq {b}: {st}")
        assert_close_bf16(h_out[b], oracle.bf16_to_f64(ref["h_out"]), f"{name} seq {b}: h_out")
        kc, vc, sm = (host_u16(t) for t in dev_caches[b])
        assert np.array_equal(kc[:, n - 1], forced["k"]) and np.array_equal(vc[:, n - 1], forced["v"])
        assert np.array_equal(sm, so), f"{name} seq {b}: block summary"


def test_batch_step_equals_layer_chain_and_head():
    """bc_decode_step_batch: its hidden states equal the chain of
    bc_decode_layer_batch calls bit for bit; its logits against the oracle's
    LM head applied to each sequence's final hidden state; tokens = argmax."""
    from activation_kv_cache_amd import binding as bc
    dims = dict(gen.TINY, vocab=1000, n_layers=2)
    d, V_ = dims["d"], dims["vocab"]
    B, n_cap, n, S = 3, 1024, 1000, 4
    md = bc.dims(dims)
    pol = bc.policy(0.3, 4, 64)
    Ws = [gen.layer_weights(82, dims, layer=li) for li in range(2)]
    pws = [_packed(W, dims) for W in Ws]
    host_caches = [_caches(dims, n_cap, n, 82, li, B, 0.5) for li in range(2)]
    g_final = gen.to_bf16_bits(np.ones(d, np.float32))
    w_head = gen.normal_bf16(82, "bhead", (d, V_), 0.02)
    gf, wh = dev(g_final), bc.packed_tiles(dev(w_head))
    h0 = np.stack([gen.activation_bf16(82, f"bh{b}", d) for b in range(B)])

    def make():
        dc = [[(dev(K), dev(V), dev(sm)) for K, V, sm in host_caches[li]] for li in range(2)]
        lys = [bc.make_layer(pws[li]["qkv"], pws[li]["o"], pws[li]["gu"], pws[li]["down"], pws[li]["g1"],
                             pws[li]["g2"], *dc[li][b]) for li in range(2) for b in range(B)]
        return dc, lys

    st = bc.make_step(n, 0.5, pol, S)
    ws = workspace(bc.bc_layer_batch_workspace_bytes(md, B, n_cap, S))
    _, lys = make()
    h1 = dev(h0)
    for li in range(2):
        bc.bc_decode_layer_batch(md, bc.make_layer_array(lys[li * B:(li + 1) * B]), st, h1, ws)
    _, lys2 = make()
    h2 = dev(h0)
    logits = torch.full((B, V_), float("nan"), dtype=torch.float32, device="cuda")
    tok = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    bc.bc_decode_step_batch(md, bc.make_layer_array(lys2), 2, B, gf, wh, st, h2, logits, tok, ws)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
    lg = host(logits)
    for b in range(B):
        _, y64, _ = oracle.lm_head(host_u16(h2)[b], g_final, w_head)
        assert_close(lg[b], y64, f"logits seq {b}")
        assert int(host(tok)[b]) == int(np.argmax(lg[b]))
