"""GPU parity of the whole decode step (bc_decode_step: every layer, the
final norm, the LM head and the argmax) against the CPU oracle's chain of
layers and its LM head (README "Timing and quality on a GPU": a step is
every layer with all seven projections and the cache read, then the LM
head).

Nothing floating-point is teacher-forced here.  With sparse keeps the oracle
takes the channel and KV index sets the GPU chose (those integer decisions
are checked bit for bit, given their inputs, by the layer tests); the step
itself is first shown bit-identical to the chain of bc_decode_layer calls
whose taps supply those sets.  Bars:
  - hidden state after the last layer: |gpu - ref| <= 2e-3 + 1e-2|ref| plus,
    per layer, the independent-rounding terms of the one-layer end-to-end
    test (one bf16 ulp of that layer's h_mid and 4 standard deviations of one
    ulp of each SwiGLU output carried through W_down), and relative L2 < 1e-2;
  - logits against the oracle's LM head applied to the GPU's own final hidden
    state: 2e-3 + 1e-2|ref| elementwise;
  - logits end to end (oracle chain + oracle LM head): relative L2 < 1e-2;
  - the argmax token is reported, not gated (random-weight logits are near
    ties)."""
import numpy as np
import pytest
import torch

import oracle
from activation_kv_cache_amd import inputs as gen

from gpu_util import assert_close, dev, host, host_u16, workspace

pytestmark = pytest.mark.gpu


def _ulp(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return 2.0 ** (np.maximum(e, -126) - 7)


def _draw(seed, name, shape, std, on_device):
    """A seeded bf16 tensor on the host: drawn by numpy, or (large ones) by
    the device generator and copied back."""
    if on_device:
        return host_u16(gen.device_normal_bf16(seed, name, shape, std))
    return gen.normal_bf16(seed, name, shape, std)


def _weights(seed, dims, li, on_device):
    d, H, Hkv, D, dff = dims["d"], dims["n_heads"], dims["n_kv_heads"], dims["head_dim"], dims["d_ff"]
    p = f"layer{li}/"
    one = gen.to_bf16_bits(np.ones(d, np.float32))
    return {"qkv": _draw(seed, p + "wqkv", (d, H * D + 2 * Hkv * D), 0.02, on_device),
            "o": _draw(seed, p + "wo", (H * D, d), 0.02, on_device),
            "gate": _draw(seed, p + "wgate", (d, dff), 0.02, on_device),
            "up": _draw(seed, p + "wup", (d, dff), 0.02, on_device),
            "down": _draw(seed, p + "wdown", (dff, d), 0.02, on_device),
            "g1": one.copy(), "g2": one.copy()}


def _case(dims, n_layers, n_cap, n, r_p, r_kv, sinks, window, S, seed, kv_std):
    from activation_kv_cache_amd import binding as bc
    d, dff, H, Hkv, D, vocab = (dims["d"], dims["d_ff"], dims["n_heads"], dims["n_kv_heads"], dims["head_dim"],
                                dims["vocab"])
    dims = dict(dims, n_layers=n_layers)
    md = bc.dims(dims)
    pol = bc.policy(r_kv, sinks, window)
    t_sel = bc.bc_kv_budget(n, pol)["t_sel"]
    S = S or bc.bc_attn_default_splits(t_sel if r_kv < 1 else n, Hkv)
    print(f"[step] dims d={d} layers={n_layers} n={n} r_p={r_p} r_kv={r_kv} S={S}", flush=True)
    big = d >= 4096
    Ws, caches, packed = [], [], []
    for li in range(n_layers):
        W = _weights(seed, dims, li, big)
        K = _draw(seed, f"layer{li}/kcache", (Hkv, n_cap, D), kv_std, big)
        V = _draw(seed, f"layer{li}/vcache", (Hkv, n_cap, D), kv_std, big)
        summ = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
        for g in range(Hkv):
            s = oracle.kv_summary(K[g], n - 1)
            summ[g, :s.shape[0]] = s
        w = {k: dev(v) for k, v in W.items()}
        w_gu = torch.empty(2 * d * dff, dtype=torch.int16, device="cuda")
        bc.bc_pack_gate_up(w["gate"], w["up"], w_gu)
        packed.append(dict(qkv=bc.packed_tiles(w["qkv"]), o=bc.packed_tiles(w["o"]), gu=w_gu,
                           down=bc.packed_tiles(w["down"]), g1=w["g1"], g2=w["g2"]))
        del w
        Ws.append(W)
        caches.append((K, V, summ))
    g_final = gen.to_bf16_bits(np.ones(d, np.float32))
    w_head = _draw(seed, "head", (d, vocab), 0.02, big)
    gf_d = dev(g_final)
    wh_d = bc.packed_tiles(dev(w_head))
    h0 = gen.activation_bf16(seed, "h0", d)

    def device_layers():
        kv = [(dev(K), dev(V), dev(sm)) for K, V, sm in caches]
        cl = [bc.make_layer(p["qkv"], p["o"], p["gu"], p["down"], p["g1"], p["g2"], *kv[i])
              for i, p in enumerate(packed)]
        return kv, cl

    # the step
    _, cl = device_layers()
    arr = bc.make_layer_array(cl)
    h_step = dev(h0)
    lg_step = torch.full((vocab,), float("nan"), dtype=torch.float32, device="cuda")
    tk_step = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    st = bc.make_step(n, r_p, pol, S)
    bc.bc_decode_step(md, arr, gf_d, wh_d, st, h_step, lg_step, tk_step,
                      workspace(bc.bc_step_workspace_bytes(md, n_cap, S)))
    torch.cuda.synchronize()

    # the same step as a chain of layer calls with taps (the index sets)
    forced = [dict() for _ in range(n_layers)]
    sparse = r_p < 1 or r_kv < 1
    if sparse:
        _, cl2 = device_layers()
        h = dev(h0)
        ws = workspace(bc.bc_layer_workspace_bytes(md, n_cap, S))
        k_d, k_ff = oracle.channel_keep(r_p, d), oracle.channel_keep(r_p, dff)
        for li, c in enumerate(cl2):
            sizes = {}
            if r_p < 1:
                sizes.update(idx_qkv=k_d, idx_o=k_d, idx_gu=k_d, idx_down=k_ff)
            if r_kv < 1:
                sizes["idx_kv"] = Hkv * t_sel
            taps = {k: torch.full((v,), -1, dtype=torch.int32, device="cuda") for k, v in sizes.items()}
            bc.bc_decode_layer(md, c, bc.make_step(n, r_p, pol, S, taps=bc.make_taps(**taps)), h, ws)
            torch.cuda.synchronize()
            for k, t in taps.items():
                forced[li][k] = host(t).reshape(Hkv, -1) if k == "idx_kv" else host(t)
        lg = torch.empty_like(lg_step)
        tk = torch.empty_like(tk_step)
        bc.bc_lm_head(md, h, gf_d, wh_d, lg, tk, 1e-5, workspace(bc.bc_lm_head_workspace_bytes(md)))
        torch.cuda.synchronize()
        assert torch.equal(h, h_step) and torch.equal(lg, lg_step) and torch.equal(tk, tk_step), \
            "bc_decode_step differs from its chain of bc_decode_layer calls"

    # the oracle's chain: no floating-point forcing
    h_ref = h0
    flips = 0
    slack = np.zeros(d)
    for li in range(n_layers):
        K, V, summ = caches[li]
        ref = oracle.decode_layer(h_ref, Ws[li], K.copy(), V.copy(), summ.copy(), n, dims, r_p, r_kv, sinks,
                                  window, S, forced=forced[li])
        for k, v in forced[li].items():
            flips += int(not np.array_equal(np.asarray(ref[k]).reshape(v.shape), v))
        wd = oracle.bf16_to_f64(Ws[li]["down"])
        uf = _ulp(oracle.bf16_to_f64(ref["hff"])).reshape(-1)
        slack += _ulp(oracle.bf16_to_f64(ref["h_mid"])).reshape(-1) + 4 * np.sqrt((wd * wd).T @ (uf * uf))
        h_ref = ref["h_out"]
    g = oracle.bf16_to_f64(host_u16(h_step)).reshape(-1)
    r = oracle.bf16_to_f64(h_ref).reshape(-1)
    err = np.abs(g - r)
    tol = 2e-3 + 1e-2 * np.abs(r) + slack
    rel = np.linalg.norm(g - r) / np.linalg.norm(r)
    print(f"[step] hidden: max err {err.max():.3g}, max err/tol {(err / tol).max():.3f}, rel-L2 {rel:.3g}; "
          f"selections the oracle would have made differently on its own: {flips}", flush=True)
    assert (err <= tol).all(), f"final hidden: {(err > tol).sum()} of {err.size} outside the bound"
    assert rel < 1e-2, f"final hidden: rel-L2 {rel:.3g}"
    # the LM head on the GPU's own final hidden state
    _, y_forced, _ = oracle.lm_head(host_u16(h_step), g_final, w_head)
    lg_g = host(lg_step)
    assert_close(lg_g, y_forced, "logits (LM head on the step's hidden state)")
    assert int(host(tk_step)[0]) == int(np.argmax(lg_g))
    # logits end to end
    _, y_ref, arg_ref = oracle.lm_head(h_ref, g_final, w_head)
    rel_lg = np.linalg.norm(lg_g - y_ref) / np.linalg.norm(y_ref)
    print(f"[step] logits end to end: rel-L2 {rel_lg:.3g}; argmax gpu {int(host(tk_step)[0])} "
          f"oracle {arg_ref} (reported, not gated)", flush=True)
    assert rel_lg < 1e-2, f"logits: rel-L2 {rel_lg:.3g}"


TINY_STEP = [
    # (name, r_p, r_kv, S)
    ("dense", 1.0, 1.0, 4),
    ("proj-0.7", 0.7, 1.0, 4),
    ("kv-0.3", 1.0, 0.3, 4),
    ("both-0.5-0.3", 0.5, 0.3, 4),
    ("both-0.5-0.5-default-splits", 0.5, 0.5, 0),
]


@pytest.mark.parametrize("name,r_p,r_kv,S", TINY_STEP, ids=[c[0] for c in TINY_STEP])
def test_step_vs_oracle_tiny(name, r_p, r_kv, S):
    """Three tiny layers (d 512, 8/2 heads, head_dim 64, d_ff 1408) at 2000
    tokens of a 2048-token cache, LM head of 1000 words."""
    _case(dict(gen.TINY, vocab=1000), 3, 2048, 2000, r_p, r_kv, 4, 128, S, seed=41, kv_std=0.5)


@pytest.mark.parametrize("r_p,r_kv", [(1.0, 1.0), (0.5, 0.3)], ids=["dense", "both-0.5-0.3"])
def test_step_vs_oracle_8b_2k(r_p, r_kv):
    """Two Llama-3.1-8B layers at 2048 tokens with the full 128256-word LM
    head, in the launch configuration of the bench (default splits, window
    1024), KV ~ N(0, 1)."""
    _case(gen.LLAMA8B, 2, 2048, 2048, r_p, r_kv, 4, 1024, 0, seed=42, kv_std=1.0)


@pytest.mark.parametrize("r_p,r_kv", [(1.0, 1.0), (0.5, 0.3)], ids=["dense", "both-0.5-0.3"])
def test_consecutive_steps_cross_a_block(r_p, r_kv):
    """Eight consecutive decode steps on one cache (tiny dims, two layers, LM
    head of 1000 words) at contexts 1020..1027: the appends (slots 1019..1026)
    cross the block boundary at 1024, each step refreshing the summary of the
    block it writes into and the next step reading both.  Per step: the step
    equals, bit for bit, the chain of bc_decode_layer calls run on a second
    copy of the caches (hidden state, logits, token), and the oracle's chain
    of layers -- on host copies of the caches, with the GPU's index sets and
    appended k, v rows -- gives the same hidden state within the single-step
    bound.  After the last step both caches, and every block summary, equal
    the oracle's; each summary also equals its definition (per dim the min
    and max over the block's rows below the context) recomputed from the
    GPU's own cache."""
    from activation_kv_cache_amd import binding as bc
    dims = dict(gen.TINY, vocab=1000, n_layers=2)
    d, dff, H, Hkv, D, vocab = (dims["d"], dims["d_ff"], dims["n_heads"], dims["n_kv_heads"], dims["head_dim"],
                                dims["vocab"])
    n_cap, n0, steps, sinks, window, S, seed = 2048, 1020, 8, 4, 128, 4, 43
    md = bc.dims(dims)
    pol = bc.policy(r_kv, sinks, window)
    Ws, host_caches = [], []
    for li in range(2):
        Ws.append(_weights(seed, dims, li, False))
        K = gen.normal_bf16(seed, f"layer{li}/kcache", (Hkv, n_cap, D), 0.5)
        V = gen.normal_bf16(seed, f"layer{li}/vcache", (Hkv, n_cap, D), 0.5)
        summ = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
        for g in range(Hkv):
            s = oracle.kv_summary(K[g], n0 - 1)
            summ[g, :s.shape[0]] = s
        host_caches.append([K, V, summ])
    g_final = gen.to_bf16_bits(np.ones(d, np.float32))
    w_head = gen.normal_bf16(seed, "head", (d, vocab), 0.02)
    gf_d, wh_d = dev(g_final), bc.packed_tiles(dev(w_head))
    packed = []
    for W in Ws:
        w = {k: dev(v) for k, v in W.items()}
        w_gu = torch.empty(2 * d * dff, dtype=torch.int16, device="cuda")
        bc.bc_pack_gate_up(w["gate"], w["up"], w_gu)
        packed.append(dict(qkv=bc.packed_tiles(w["qkv"]), o=bc.packed_tiles(w["o"]), gu=w_gu,
                           down=bc.packed_tiles(w["down"]), g1=w["g1"], g2=w["g2"]))

    def device_copy():
        kv = [(dev(K), dev(V), dev(sm)) for K, V, sm in host_caches]
        return kv, [bc.make_layer(p["qkv"], p["o"], p["gu"], p["down"], p["g1"], p["g2"], *kv[i])
                    for i, p in enumerate(packed)]

    kv_a, cl_a = device_copy()     # the step's caches
    kv_b, cl_b = device_copy()     # the layer chain's caches
    arr = bc.make_layer_array(cl_a)
    ws_step = workspace(bc.bc_step_workspace_bytes(md, n_cap, S))
    ws_layer = workspace(bc.bc_layer_workspace_bytes(md, n_cap, S))
    ws_head = workspace(bc.bc_lm_head_workspace_bytes(md))
    k_d, k_ff = oracle.channel_keep(r_p, d), oracle.channel_keep(r_p, dff)
    for t in range(steps):
        n = n0 + t
        t_sel = bc.bc_kv_budget(n, pol)["t_sel"]
        h0 = gen.activation_bf16(seed, f"h{t}", d)
        h_a = dev(h0)
        lg_a = torch.full((vocab,), float("nan"), dtype=torch.float32, device="cuda")
        tk_a = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        bc.bc_decode_step(md, arr, gf_d, wh_d, bc.make_step(n, r_p, pol, S), h_a, lg_a, tk_a, ws_step)
        h_b = dev(h0)
        forced = []
        for c in cl_b:
            sizes = {"k": Hkv * D, "v": Hkv * D}
            if r_p < 1:
                sizes.update(idx_qkv=k_d, idx_o=k_d, idx_gu=k_d, idx_down=k_ff)
            if r_kv < 1:
                sizes["idx_kv"] = Hkv * t_sel
            taps = {k: torch.full((v,), -1, dtype=torch.int16 if k in ("k", "v") else torch.int32, device="cuda")
                    for k, v in sizes.items()}
            bc.bc_decode_layer(md, c, bc.make_step(n, r_p, pol, S, taps=bc.make_taps(**taps)), h_b, ws_layer)
            torch.cuda.synchronize()
            f = {}
            for k, tv in taps.items():
                if k in ("k", "v"):
                    f[k] = host_u16(tv).reshape(Hkv, D)
                else:
                    f[k] = host(tv).reshape(Hkv, -1) if k == "idx_kv" else host(tv)
            forced.append(f)
        lg_b = torch.empty_like(lg_a)
        tk_b = torch.empty_like(tk_a)
        bc.bc_lm_head(md, h_b, gf_d, wh_d, lg_b, tk_b, 1e-5, ws_head)
        torch.cuda.synchronize()
        assert torch.equal(h_a, h_b) and torch.equal(lg_a, lg_b) and torch.equal(tk_a, tk_b), \
            f"step {t}: bc_decode_step differs from its chain of bc_decode_layer calls"
        # the oracle's chain on its own caches (updated in place)
        h_ref = h0
        slack = np.zeros(d)
        for li in range(2):
            K, V, summ = host_caches[li]
            ref = oracle.decode_layer(h_ref, Ws[li], K, V, summ, n, dims, r_p, r_kv, sinks, window, S,
                                      forced=forced[li])
            wd = oracle.bf16_to_f64(Ws[li]["down"])
            uf = _ulp(oracle.bf16_to_f64(ref["hff"])).reshape(-1)
            slack += _ulp(oracle.bf16_to_f64(ref["h_mid"])).reshape(-1) + 4 * np.sqrt((wd * wd).T @ (uf * uf))
            h_ref = ref["h_out"]
        g = oracle.bf16_to_f64(host_u16(h_a)).reshape(-1)
        r = oracle.bf16_to_f64(h_ref).reshape(-1)
        err = np.abs(g - r)
        assert (err <= 2e-3 + 1e-2 * np.abs(r) + slack).all(), f"step {t} (context {n}): hidden outside the bound"
        assert np.linalg.norm(g - r) / np.linalg.norm(r) < 1e-2
    n_last = n0 + steps - 1
    nb = (n_last + 15) // 16
    for li in range(2):
        K, V, summ = host_caches[li]
        Ka, Va, Sa = (host_u16(x) for x in kv_a[li])
        Kb, Vb, Sb = (host_u16(x) for x in kv_b[li])
        assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb) and np.array_equal(Sa, Sb), f"layer {li}: caches"
        assert np.array_equal(Ka, K) and np.array_equal(Va, V), f"layer {li}: cache rows differ from the oracle's"
        assert np.array_equal(Sa[:, :nb], summ[:, :nb]), f"layer {li}: summaries differ from the oracle's"
        for g in range(Hkv):   # as values (a refresh meets the new row first: -0 and +0 may swap)
            assert np.array_equal(oracle.bf16_to_f64(Sa[g, :nb]), oracle.bf16_to_f64(oracle.kv_summary(Ka[g], n_last))), \
                f"layer {li} head {g}: summary"
