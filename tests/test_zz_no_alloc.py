"""bc_decode_step_noalloc (the step with the library's static workspace)
against bc_decode_step with a caller workspace: same bits, on two calls in a
row, the second with a smaller context and other keeps."""
import numpy as np
import pytest
import torch

import oracle
from activation_kv_cache_amd import inputs as gen

from gpu_util import dev, workspace

pytestmark = pytest.mark.gpu


def _model(dims, n_cap, seed):
    from activation_kv_cache_amd import binding as bc
    d, dff, Hkv, D = dims["d"], dims["d_ff"], dims["n_kv_heads"], dims["head_dim"]
    layers, caches = [], []
    for li in range(dims["n_layers"]):
        W = gen.layer_weights(seed, dims, layer=li)
        w = {k: dev(v) for k, v in W.items()}
        w_gu = torch.empty(2 * d * dff, dtype=torch.int16, device="cuda")
        bc.bc_pack_gate_up(w["gate"], w["up"], w_gu)
        K, V = gen.kv_cache(seed, dims, n_cap, 0.5, layer=li)
        layers.append(dict(qkv=bc.packed_tiles(w["qkv"]), o=bc.packed_tiles(w["o"]), gu=w_gu,
                           down=bc.packed_tiles(w["down"]), g1=w["g1"], g2=w["g2"]))
        caches.append((K, V))
    g_final = dev(gen.to_bf16_bits(np.ones(d, np.float32)))
    w_head = bc.packed_tiles(dev(gen.normal_bf16(seed, "head", (d, dims["vocab"]), 0.02)))
    return layers, caches, g_final, w_head


def _fresh(layers, caches, n, dims):
    """Device caches (pre-filled below n) with their block summaries, and the
    layer structs over them."""
    from activation_kv_cache_amd import binding as bc
    Hkv, D = dims["n_kv_heads"], dims["head_dim"]
    kv = []
    for K, V in caches:
        n_cap = K.shape[1]
        summ = np.zeros((Hkv, n_cap // 16, D, 2), np.uint16)
        for g in range(Hkv):
            t = oracle.kv_summary(K[g], n - 1)
            summ[g, :t.shape[0]] = t
        kv.append((dev(K), dev(V), dev(summ)))
    cl = [bc.make_layer(l["qkv"], l["o"], l["gu"], l["down"], l["g1"], l["g2"], *kv[i])
          for i, l in enumerate(layers)]
    return kv, bc.make_layer_array(cl)


def test_noalloc_step_equals_step_with_workspace():
    from activation_kv_cache_amd import binding as bc
    dims = dict(gen.TINY, vocab=1000, n_layers=3)
    n_cap = 1024
    layers, caches, g_final, w_head = _model(dims, n_cap, 31)
    md = bc.dims(dims)
    h0 = gen.activation_bf16(31, "h0", dims["d"])
    # two calls in a row on the same device: the second with a smaller
    # context, so a smaller workspace, over what the first one left
    for n, r_p, r_kv, S in ((1000, 0.5, 0.3, 4), (300, 0.7, 1.0, 0)):
        st = bc.make_step(n, r_p, bc.policy(r_kv, 4, 64), S)
        out = []
        for which in ("ws", "noalloc"):
            kv, arr = _fresh(layers, caches, n, dims)
            h = dev(h0)
            lg = torch.full((dims["vocab"],), float("nan"), dtype=torch.float32, device="cuda")
            tk = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            print(f"[noalloc] n={n} r_p={r_p} r_kv={r_kv} S={S} path={which}", flush=True)
            if which == "ws":
                ws = workspace(bc.bc_step_workspace_bytes(md, n_cap, max(S, 1) if S else 64))
                bc.bc_decode_step(md, arr, g_final, w_head, st, h, lg, tk, ws)
            else:
                bc.bc_decode_step_noalloc(md, arr, g_final, w_head, st, h, lg, tk)
            torch.cuda.synchronize()
            out.append((h, lg, tk, kv))
        (h1, lg1, tk1, kv1), (h2, lg2, tk2, kv2) = out
        assert torch.isfinite(lg1).all()
        assert torch.equal(h1, h2), n
        assert torch.equal(lg1, lg2), n
        assert torch.equal(tk1, tk2), n
        for a, b in zip(kv1, kv2):
            for x, y in zip(a, b):
                assert torch.equal(x, y), n
