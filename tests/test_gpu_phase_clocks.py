"""The instrumented build (libbc_clk.so: the library's kernels plus shader-
clock reads at phase ends) computes what the library computes: a tiny
two-layer decode step, dense and composed (r_p 0.5, r_kv 0.3), run in a
process of its own under each build, gives bit-identical hidden states,
logits and tokens; and the clocks it records are well formed (every GEMV
and attention launch of the step recorded, every work-group's stamps in
order).  Skipped when the instrumented build is not there."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "activation_kv_cache_amd")

SCRIPT = r'''
import json, os, sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from activation_kv_cache_amd import binding as bc
from activation_kv_cache_amd import inputs as gen
out_dir = sys.argv[2]
D = dict(gen.TINY, n_layers=2)
d, dff, H, Hkv, hd = D["d"], D["d_ff"], D["n_heads"], D["n_kv_heads"], D["head_dim"]
n_cap = n = 2048
md = bc.dims(D)
one = torch.full((d,), 1.0, dtype=torch.bfloat16, device="cuda").view(torch.int16)
keep = []
layers = []
for li in range(2):
    p = f"layer{li}/"
    w_qkv = bc.packed_tiles(gen.device_normal_bf16(7, p + "wqkv", (d, H * hd + 2 * Hkv * hd), 0.02))
    w_o = bc.packed_tiles(gen.device_normal_bf16(7, p + "wo", (H * hd, d), 0.02))
    gate = gen.device_normal_bf16(7, p + "wgate", (d, dff), 0.02)
    up = gen.device_normal_bf16(7, p + "wup", (d, dff), 0.02)
    w_gu = torch.empty(2 * d * dff, dtype=torch.int16, device="cuda")
    bc.bc_pack_gate_up(gate, up, w_gu)
    w_down = bc.packed_tiles(gen.device_normal_bf16(7, p + "wdown", (dff, d), 0.02))
    k = gen.device_normal_bf16(7, p + "k", (Hkv, n_cap, hd), 1.0)
    v = gen.device_normal_bf16(7, p + "v", (Hkv, n_cap, hd), 1.0)
    summ = torch.empty((Hkv, n_cap // 16, hd, 2), dtype=torch.int16, device="cuda")
    bc.bc_build_kv_summary(k, n - 1, summ)
    keep += [w_qkv, w_o, w_gu, w_down, k, v, summ]
    layers.append(bc.make_layer(w_qkv, w_o, w_gu, w_down, one, one, k, v, summ))
arr = bc.make_layer_array(layers)
w_head = bc.packed_tiles(gen.device_normal_bf16(7, "head", (d, D["vocab"]), 0.02))
h0 = torch.from_numpy(gen.activation_bf16(7, "h0", d).view(np.int16)).cuda()
ws = torch.empty(bc.bc_step_workspace_bytes(md, n_cap, 64) // 4 + 64, dtype=torch.int32, device="cuda")
bc.bc_workspace_init(ws)
clocks = bc.LIB_NAME == "libbc_clk.so"
buf = torch.zeros(1 << 20, dtype=torch.int64, device="cuda")
report = {"library": bc.LIB_NAME}
for tag, r_p, r_kv in (("dense", 1.0, 1.0), ("both", 0.5, 0.3)):
    pol = bc.policy(r_kv, 4, 128)
    st = bc.make_step(n, r_p, pol, 8)
    h = h0.clone()
    logits = torch.empty(D["vocab"], dtype=torch.float32, device="cuda")
    token = torch.empty(1, dtype=torch.int32, device="cuda")
    # the saved state of the caches: the step appends at slot n - 1
    saved = [t.clone() for t in keep]
    if clocks:
        buf.zero_()
        bc.bc_phase_clocks_begin(buf)
    bc.bc_decode_step(md, arr, one, w_head, st, h, logits, token, ws)
    torch.cuda.synchronize()
    if clocks:
        launches = bc.bc_phase_clocks_launches()
        bc.bc_phase_clocks_begin(None)
        clk = buf.cpu().numpy()
        ok = True
        kinds = {1: 0, 2: 0}
        for (kind, a, b, c, dd, groups, off) in launches:
            kinds[kind] += 1
            t = clk[off: off + 16 * groups].reshape(groups, 16)
            ok &= bool(((t[:, 1] > t[:, 0]) & (t[:, 13] > t[:, 2])).all())
            for i in range(3, 13):
                sel = t[:, i] > 0
                ok &= bool(((t[sel, i] >= t[sel, 2]) & (t[sel, i] <= t[sel, 13])).all())
        report[tag] = {"gemv_launches": kinds[1], "attn_launches": kinds[2], "stamps_in_order": ok}
    np.save(os.path.join(out_dir, f"{tag}_h.npy"), h.cpu().numpy())
    np.save(os.path.join(out_dir, f"{tag}_logits.npy"), logits.cpu().numpy())
    np.save(os.path.join(out_dir, f"{tag}_token.npy"), token.cpu().numpy())
    for t, s in zip(keep, saved):
        t.copy_(s)
json.dump(report, open(os.path.join(out_dir, "report.json"), "w"))
print("[phase-clocks] done", bc.LIB_NAME, flush=True)
'''


def _run(lib, out_dir):
    env = dict(os.environ, BC_LIBRARY=lib)
    print(f"[phase-clocks] tiny step under {lib}", flush=True)
    r = subprocess.run([sys.executable, "-c", SCRIPT, ROOT, str(out_dir)], env=env, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    return json.load(open(os.path.join(out_dir, "report.json")))


@pytest.mark.skipif(not os.path.exists(os.path.join(PKG, "libbc_clk.so")), reason="libbc_clk.so not built")
def test_instrumented_build_computes_the_same_step(tmp_path):
    a, b = tmp_path / "lib", tmp_path / "clk"
    a.mkdir()
    b.mkdir()
    rep_a = _run("libbc.so", a)
    rep_b = _run("libbc_clk.so", b)
    assert rep_a["library"] == "libbc.so" and rep_b["library"] == "libbc_clk.so"
    for tag in ("dense", "both"):
        for what in ("h", "logits", "token"):
            x = np.load(a / f"{tag}_{what}.npy")
            y = np.load(b / f"{tag}_{what}.npy")
            assert x.tobytes() == y.tobytes(), (tag, what)
        r = rep_b[tag]
        # per layer: q/k/v, o, gate|up, down GEMVs and one attention partial launch, then the LM head
        assert r["gemv_launches"] == 2 * 4 + 1, r
        assert r["attn_launches"] == 2, r
        assert r["stamps_in_order"], r
