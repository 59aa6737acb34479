#!/usr/bin/env python3
"""Decode-step benchmark at Llama-3.1-8B dimensions on one MI355X.

A step is one full decode step of one sequence: 32 x bc_decode_layer
(activation-sparse projection GEMVs and split-K attention over the KV cache,
read densely or through the scored selection) + final RMSNorm + dense LM
head + argmax, captured once as a HIP graph and replayed.  Weights are random
N(0, 0.02), the KV cache N(0, 1) pre-filled to 131072 tokens, the hidden
input N(0, 1) with 1% outlier channels x10; all drawn on the device from
seeded generators.  The context is held fixed: every step writes the new
token at slot n-1 again.

The headline line is the dense step at 131072 tokens (r_p = r_kv = 1):
value = algorithmic bytes of the step / step time.  The other cells (modes
and contexts) are reported under "cells".  Algorithmic bytes per step:
  r_p-weighted projection weights + LM head + 4096 B x L x T_sel (K and V)
  + [KV selection] 256 B x L x n (block summaries) + index lists, partials.
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-step µs and achieved HBM GB/s vs context 2K–128K, Llama-3.1-8B dims"
HBM_PEAK_GBS = 8000.0
DIMS = dict(n_layers=32, d=4096, d_ff=14336, vocab=128256, n_heads=32, n_kv_heads=8, head_dim=128)
SINKS, WINDOW = 4, 1024
W_OBS, POOL = 32, 5       # select-once (SnapKV form): observation window, pooling kernel
KERNEL_SOURCES = ["activation_kv_cache_amd/csrc/bc_attn.hip", "activation_kv_cache_amd/csrc/bc_device.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ byte account
def channel_keep(r_p, n):
    return n if r_p >= 1 else max(1, min(n, int(math.floor(r_p * n + 0.5))))


def gemv_bytes(d_in, d_out, k, sparse):
    b = 2 * k * d_out + 2 * d_out + 2 * (k if sparse else d_in)
    return b + (4 * k if sparse else 0)


def attn_bytes(n_sel, S, sparse):
    D = DIMS
    kv = 2 * D["n_kv_heads"] * D["head_dim"] * 2 * n_sel
    part = D["n_heads"] * S * (D["head_dim"] + 2) * 4
    return kv + part + (4 * D["n_kv_heads"] * n_sel if sparse else 0)


def layer_bytes(n, r_p, r_kv, t_sel, S, scored=True):
    """Algorithmic bytes of one layer.  scored=False is the KV-window
    baseline: the kept tokens are the sinks and the most recent ones, so no
    summaries are scored and no index list is written or read."""
    D = DIMS
    d, dff, H, Hkv, hd = D["d"], D["d_ff"], D["n_heads"], D["n_kv_heads"], D["head_dim"]
    sp = r_p < 1
    kd, kf = channel_keep(r_p, d), channel_keep(r_p, dff)
    b = gemv_bytes(d, H * hd + 2 * Hkv * hd, kd, sp)
    b += gemv_bytes(H * hd, d, kd, sp)
    b += gemv_bytes(d, 2 * dff, kd, sp)
    b += gemv_bytes(dff, d, kf, sp)
    b += attn_bytes(t_sel, S, r_kv < 1 and scored)
    if r_kv < 1 and scored:
        b += 2 * Hkv * hd * 2 * ((n + 15) // 16) + 4 * Hkv * t_sel
    return b


def step_bytes(n, r_p, r_kv, t_sel, S, scored=True):
    D = DIMS
    return D["n_layers"] * layer_bytes(n, r_p, r_kv, t_sel, S, scored) + 2 * D["d"] * D["vocab"] + 4 * D["vocab"]


def byte_bound(n, r_p, r_kv):
    """Ideal speedup of a mode over dense decoding from bytes alone (README
    "Quick start", bound): B / (B - dB) with B the projection weights, LM
    head and K and V bytes of the step and dB the bytes the two branches
    skip; summaries, index lists and activations are left out."""
    D = DIMS
    kvd = D["n_kv_heads"] * D["head_dim"]
    w_proj = 2 * D["n_layers"] * (2 * D["d"] ** 2 + 2 * D["d"] * kvd + 3 * D["d"] * D["d_ff"])
    B = w_proj + 2 * D["vocab"] * D["d"] + 2 * 2 * D["n_layers"] * kvd * n
    dB = (1 - r_p) * w_proj + (1 - r_kv) * 2 * 2 * D["n_layers"] * kvd * n
    return B / (B - dB)


def n_star_k(r_p, r_kv, ext=False):
    """Context (in units of 1024 tokens) at which skipping (1 - r_p) of the
    projection weights and (1 - r_kv) of the K and V bytes save the same
    bytes per step (README "Quick start" / "Usage": the byte crossover).
    ext also charges the KV branch the block summaries it scores every step
    (1/16 of the K and V bytes)."""
    D = DIMS
    kvd = D["n_kv_heads"] * D["head_dim"]
    w_proj = 2 * D["n_layers"] * (2 * D["d"] ** 2 + 2 * D["d"] * kvd + 3 * D["d"] * D["d_ff"])
    kv_per_token = 2 * 2 * D["n_layers"] * kvd
    return (1 - r_p) * w_proj / ((1 - r_kv - (1.0 / 16 if ext else 0.0)) * kv_per_token) / 1024


def batch_crossover_k(union_keep, r_kv, batch):
    """Byte crossover of a batch (README "Quick start", crossover_batch): the
    projection weights are read once for the union of the batch's channel
    lists (union_keep of them), the K and V bytes once per sequence; in
    units of 1024 tokens."""
    D = DIMS
    kvd = D["n_kv_heads"] * D["head_dim"]
    w_proj = 2 * D["n_layers"] * (2 * D["d"] ** 2 + 2 * D["d"] * kvd + 3 * D["d"] * D["d_ff"])
    kv_per_token = 2 * 2 * D["n_layers"] * kvd
    return (1 - union_keep) * w_proj / ((1 - r_kv) * batch * kv_per_token) / 1024


def batch_gemv_bytes(n_union, d_in, d_out, k, batch):
    """Algorithmic bytes of one batched GEMV: the union's weight rows once,
    plus every sequence's input, channel list and output."""
    return 2 * n_union * d_out + batch * (2 * d_in + 4 * k + 2 * d_out)


def crossing_k(contexts, d_vals):
    """Where d = S_proj - S_kv changes sign from + to -: the last context with
    d > 0 and the next one, interpolated linearly (in units of 1024 tokens);
    None when d never turns negative after being positive."""
    for i in range(len(contexts) - 1):
        if d_vals[i] > 0 and d_vals[i + 1] <= 0 and all(x > 0 for x in d_vals[:i + 1]):
            na, nb, da, db = contexts[i], contexts[i + 1], d_vals[i], d_vals[i + 1]
            return (na + (nb - na) * da / (da - db)) / 1024
    return None


def block_resamples(blocks):
    """Every ordered draw of `blocks` blocks with replacement (blocks**blocks
    of them: 256 for four blocks, 3,125 for five), as the paper's timing
    intervals enumerate them (README "Reproduce the paper", conventions)."""
    return np.array(list(itertools.product(range(blocks), repeat=blocks)), dtype=np.int64)


def resample_intervals(t, contexts, pairs, level=0.95):
    """Block-resampled intervals of the paired speedups and of each pair's
    crossing.  t[mode] holds step times [blocks][contexts]; every resample
    averages the per-block paired speedups t_dense / t_mode over its drawn
    blocks, and its crossing is crossing_k of the averaged S_proj - S_kv.
    The interval is the central `level` percentile range over all resamples
    (linear interpolation); resamples whose difference never changes sign
    are counted, not placed.  Returns (speedup intervals per mode, crossing
    intervals per pair key)."""
    B = next(iter(t.values())).shape[0]
    draws = block_resamples(B)
    q = (50 * (1 - level), 50 * (1 + level))
    sp = {m: np.asarray(t["dense"], float) / np.asarray(t[m], float) for m in t if m != "dense"}
    speed = {}
    for m, s in sp.items():
        means = s[draws].mean(axis=1)        # [resamples][contexts]
        lo, hi = np.percentile(means, q, axis=0)
        speed[m] = {"lo": [round(float(x), 4) for x in lo], "hi": [round(float(x), 4) for x in hi]}
    cross = {}
    for key, mp, mk in pairs:
        d = (sp[mp] - sp[mk])[draws].mean(axis=1)
        cs = [crossing_k(contexts, [float(x) for x in row]) for row in d]
        got = np.array([c for c in cs if c is not None], float)
        rec = {"resamples": len(cs), "no_crossing": len(cs) - len(got), "level": level}
        if len(got):
            lo, hi = np.percentile(got, q)
            rec.update(lo_k=round(float(lo), 2), hi_k=round(float(hi), 2))
        cross[key] = rec
    return speed, cross


def kv_plan(n, r_kv, sinks=SINKS, window=WINDOW, block=16):
    """(T_sel, attention splits) of the per-step KV policy at context n, as
    the library's budget and default split rule compute them (host-only
    replica for the byte account of contexts that were not run)."""
    D = DIMS
    if r_kv >= 1:
        t_sel = n
    else:
        T = min(n, int(math.floor(r_kv * n + 0.5)))
        s = min(sinks, T)
        w = min(window, T - s)
        b_lo, b_hi = (s + block - 1) // block, (n - w) // block
        k_blk = min((T - s - w) // block, max(0, b_hi - b_lo))
        t_sel = s + w + block * k_blk
    splits = max(1, min(256 // D["n_kv_heads"], -(-t_sel // 64)))
    return t_sel, splits


def snap_t_sel(n, r_kv):
    """Tokens kept by the select-once policy: T = min(n, floor(r_kv n + 1/2))
    (host replica of bc_kv_snap_t_sel)."""
    return n if r_kv >= 1 else min(n, int(math.floor(r_kv * n + 0.5)))


def mode_bytes(mode, n, plan=None):
    """Algorithmic bytes of one step of a sweep mode at context n.  The sel
    modes (selection made once and gathered, README "Timing and quality on a
    GPU") step densely over the T_sel kept tokens; the kv modes read the T_sel
    listed tokens plus the block summaries they rescore every step."""
    plan = plan or (lambda n_, a, b: kv_plan(n_, b))
    r_p, r_kv, once = SWEEP_MODES[mode]
    if once:
        t_sel = snap_t_sel(n, r_kv)
        return step_bytes(t_sel, r_p, 1.0, *plan(t_sel, 1.0, 1.0))
    return step_bytes(n, r_p, r_kv, *plan(n, r_p, r_kv))


def predicted_crossing_k(contexts, t_us, mode_p, mode_k, plan=None):
    """README "Results", paper Table 2 (column Pred.): the
    byte account plus each branch's kernel cost, taken from its own sweep.
    Reading: a mode's step time is T_m(n) = B_m(n) / BW + C_m, with B_m the
    step's algorithmic bytes (mode_bytes), BW and the dense cost C_dense from
    a least-squares line through the dense cells, and C_m the mean over the
    swept contexts of T_m(n) - B_m(n) / BW.  The predicted crossing is the
    first context on a 256-token grid where the projection branch stops
    leading (T_kv - T_p turns from positive to non-positive), interpolated
    linearly; in units of 1024 tokens, None if that does not happen below
    512K tokens.  Returns (pred_k, bw_gbs, cost_p_us, cost_k_us)."""
    B = {m: np.array([mode_bytes(m, n, plan) for n in contexts], float) for m in ("dense", mode_p, mode_k)}
    td = np.asarray(t_us["dense"], float)
    slope, c_dense = np.polyfit(B["dense"], td, 1)    # us per byte, us
    cost = {m: float(np.mean(np.asarray(t_us[m], float) - B[m] * slope)) for m in (mode_p, mode_k)}

    def t_pred(m, n):
        return mode_bytes(m, n, plan) * slope + cost[m]

    prev = None
    for n in range(256, 512 * 1024 + 1, 256):
        d = t_pred(mode_k, n) - t_pred(mode_p, n)   # > 0 while the projection branch leads
        if prev is not None and prev[1] > 0 and d <= 0:
            n0, d0 = prev
            return (n0 + 256 * d0 / (d0 - d)) / 1024, 1e-3 / slope, cost[mode_p], cost[mode_k]
        prev = (n, d)
    return None, 1e-3 / slope, cost[mode_p], cost[mode_k]


COMPACT_LIMIT = 4000     # bytes of the last stdout line (a reader that keeps only the end of stdout gets it whole)


def _cell_str(c):
    pol = "" if c["r_kv"] >= 1 else (" win" if c.get("kv_policy") == "window" else " kv")
    sp = c.get("speedup_vs_dense")
    return (f"{c['r_p']}/{c['r_kv']}{pol}@{c['context']}: {c['step_us']}us {100 * c['frac_hbm']:.1f}%"
            + ("" if sp is None else f" {sp}x") + f" L{c['layer_us']}us")


def kernel_fractions(rows):
    """Each hot kernel's fraction of the 8 TB/s peak from the kernel table,
    next to the 70% target: the GEMVs (q/k/v, o, gate|up, down) dense and at
    r_p 0.5, attention dense and at r_kv 0.3 per context (with the fraction
    of the streaming-read probe at its size)."""
    res = {"target": 0.7}
    names = {"w_qkv": "qkv", "w_o": "o", "w_gu": "gu", "w_down": "down"}
    for r in rows:
        k = r.get("kernel", "")
        if r.get("gbs") is None:
            continue
        frac = round(r["gbs"] / HBM_PEAK_GBS, 3)
        if k.startswith("gemv "):
            which, rp = k.split()[1], k.split("r_p=")[1]
            if rp in ("1.0", "0.5"):
                res.setdefault(f"gemv_r_p_{rp}", {})[names.get(which, which)] = frac
        elif k == "attn_partial dense" or k == "attn_partial r_kv=0.3":
            tag = "dense" if "dense" in k else "kv0.3"
            res.setdefault("attn", {})[f"{tag}@{r['context']}"] = [frac, r.get("frac_of_probe")]
    return res


def compact_record(out, limit=COMPACT_LIMIT):
    """The record's headline fields plus one-line summaries of the cells and
    the crossings, as one JSON object of at most `limit` bytes (the full
    record is written to a file).  Optional summaries are dropped, largest
    first, until the line fits."""
    keep = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
            "vs_baseline", "dtype", "data", "config")
    c = {k: out[k] for k in keep if k in out}
    rf = out.get("roofline") or {}
    c["roofline"] = {k: rf.get(k) for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                            "launch_us", "bytes_per_launch")}
    cb = out.get("cpu_baseline")
    c["cpu_baseline"] = None if not cb else {k: cb.get(k) for k in ("value", "unit", "cores", "kind", "sample")}
    opt = {}
    if out.get("read_probe"):
        opt["read_probe"] = {k: out["read_probe"].get(k) for k in ("gbs", "frac_of_peak", "attention_frac_of_probe")}
    if out.get("cells"):
        opt["cells"] = [_cell_str(x) for x in out["cells"]]
    if out.get("gemv_roofline"):
        g = out["gemv_roofline"]
        opt["gemv_gate_up_frac"] = {k: g[k]["frac"] for k in ("dense", "r_p_0.5") if k in g}
    if out.get("kernels"):
        opt["kernel_frac"] = kernel_fractions(out["kernels"])
    for key in ("step_bytes", "masked_baseline", "batch_step", "prediction", "composed"):
        if out.get(key) and isinstance(out[key], dict) and out[key].get("summary") is not None:
            opt[key] = out[key]["summary"]
    cr = out.get("crossover")
    if cr and cr.get("pairs"):
        # per pair: [measured, interval lo, hi, n*, n*_ext, prediction] in K tokens
        opt["crossings_k"] = {k: [p.get("measured_k"), p.get("measured_interval", {}).get("lo_k"),
                                  p.get("measured_interval", {}).get("hi_k"), p.get("n_star_k"),
                                  p.get("n_star_ext_k"), p.get("pred_k")] for k, p in cr["pairs"].items()}
        sp = cr.get("speedup", {})
        ctx = cr.get("contexts", [])
        if 131072 in ctx:
            i = ctx.index(131072)
            opt["speedup_128k"] = {m: v[i] for m, v in sp.items()}
    if out.get("record_file"):
        opt["record_file"] = out["record_file"]
    c.update(opt)
    drop = ["cells", "speedup_128k", "gemv_gate_up_frac", "read_probe", "batch_step", "composed", "masked_baseline",
            "kernel_frac", "step_bytes", "prediction", "crossings_k"]
    line = json.dumps(c, separators=(",", ":"))
    while len(line.encode()) > limit and drop:
        c.pop(drop.pop(0), None)
        line = json.dumps(c, separators=(",", ":"))
    if len(line.encode()) > limit and c.get("cpu_baseline"):
        c["cpu_baseline"]["sample"] = c["cpu_baseline"]["sample"][:200]
        line = json.dumps(c, separators=(",", ":"))
    return line


def code_text(path):
    """A source file's code without its comments and white space: counters
    taken on a kernel stay valid across edits of its comments only."""
    src = open(path, encoding="utf-8").read()
    out, i, n = [], 0, len(src)
    while i < n:
        ch = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif ch in "\"'":
            j = i + 1
            while j < n and src[j] != ch:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            if not ch.isspace():
                out.append(ch)
            i += 1
    return "".join(out)


def kernel_source_hash():
    """Hash of the attention kernel's code (bc_attn.hip, bc_device.hpp),
    comments and white space left out."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(code_text(os.path.join(ROOT, f)).encode())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------- model
class Model:
    def __init__(self, max_ctx, seed=0):
        from activation_kv_cache_amd import binding as bc
        from activation_kv_cache_amd import inputs as gen

        self.bc = bc
        D = DIMS
        d, dff, H, Hkv, hd, L = D["d"], D["d_ff"], D["n_heads"], D["n_kv_heads"], D["head_dim"], D["n_layers"]
        self.max_ctx = max_ctx
        self.masked_ws = None
        self.md = bc.dims(D)
        t0 = time.time()
        one = torch.full((d,), 1.0, dtype=torch.bfloat16, device="cuda").view(torch.int16)
        self.g_attn, self.g_mlp, self.g_final = one, one.clone(), one.clone()
        self.layers = []
        for li in range(L):
            p = f"layer{li}/"
            w_qkv = bc.packed_tiles(gen.device_normal_bf16(seed, p + "wqkv", (d, H * hd + 2 * Hkv * hd), 0.02))
            w_o = bc.packed_tiles(gen.device_normal_bf16(seed, p + "wo", (H * hd, d), 0.02))
            gate = gen.device_normal_bf16(seed, p + "wgate", (d, dff), 0.02)
            up = gen.device_normal_bf16(seed, p + "wup", (d, dff), 0.02)
            w_gu = torch.empty(2 * d * dff, dtype=torch.int16, device="cuda")
            bc.bc_pack_gate_up(gate, up, w_gu)
            del gate, up
            w_down = bc.packed_tiles(gen.device_normal_bf16(seed, p + "wdown", (dff, d), 0.02))
            k = gen.device_normal_bf16(seed, p + "kcache", (Hkv, max_ctx, hd), 1.0)
            v = gen.device_normal_bf16(seed, p + "vcache", (Hkv, max_ctx, hd), 1.0)
            summ = torch.empty((Hkv, max_ctx // 16, hd, 2), dtype=torch.int16, device="cuda")
            bc.bc_build_kv_summary(k, max_ctx, summ)
            self.layers.append(dict(w_qkv=w_qkv, w_o=w_o, w_gu=w_gu, w_down=w_down, k=k, v=v, summ=summ))
        self.shapes = {"w_qkv": (d, H * hd + 2 * Hkv * hd), "w_o": (H * hd, d), "w_gu": (d, 2 * dff),
                       "w_down": (dff, d)}
        self.w_head = bc.packed_tiles(gen.device_normal_bf16(seed, "lm_head", (d, D["vocab"]), 0.02))
        h0 = gen.activation_bf16(seed, "h0", d)
        self.h0 = torch.from_numpy(h0.view(np.int16)).cuda()
        self.h = torch.empty_like(self.h0)
        self.logits = torch.empty(D["vocab"], dtype=torch.float32, device="cuda")
        self.token = torch.empty(1, dtype=torch.int32, device="cuda")
        self.ws = torch.empty(bc.bc_step_workspace_bytes(self.md, max_ctx, 1024) // 4 + 64, dtype=torch.int32,
                              device="cuda")
        self.ws_head = torch.empty(bc.bc_lm_head_workspace_bytes(self.md) // 4 + 64, dtype=torch.int32,
                                   device="cuda")
        bc.bc_workspace_init(self.ws)
        bc.bc_workspace_init(self.ws_head)
        self.c_layers = [bc.make_layer(l["w_qkv"], l["w_o"], l["w_gu"], l["w_down"], self.g_attn, self.g_mlp,
                                       l["k"], l["v"], l["summ"]) for l in self.layers]
        self.layer_array = bc.make_layer_array(self.c_layers)
        # sel modes: per layer a compact cache for the gathered selection
        # (the largest T_sel of the sweep, r_kv 0.5 at max_ctx) and the
        # observation window the selection is scored with: the post-rotary
        # queries of the last W_OBS pre-filled positions (seeded; they stand
        # in for the queries of a prefill of real text)
        cap = (snap_t_sel(max_ctx, 0.5) + 16 + 15) // 16 * 16
        self.sel_cap = cap
        self.sel_q = [gen.device_normal_bf16(seed, f"layer{li}/selq", (W_OBS, H, hd), 1.0) for li in range(L)]
        self.sel_kv = [(torch.empty((Hkv, cap, hd), dtype=torch.int16, device="cuda"),
                        torch.empty((Hkv, cap, hd), dtype=torch.int16, device="cuda")) for _ in range(L)]
        self.c_layers_sel = [bc.make_layer(l["w_qkv"], l["w_o"], l["w_gu"], l["w_down"], self.g_attn, self.g_mlp,
                                           kc, vc, None) for l, (kc, vc) in zip(self.layers, self.sel_kv)]
        self.layer_array_sel = bc.make_layer_array(self.c_layers_sel)
        self.sel_idx = torch.empty((Hkv, max_ctx), dtype=torch.int32, device="cuda")
        self.sel_ws = torch.empty(bc.bc_kv_snap_select_workspace_bytes(max_ctx, H, Hkv, W_OBS) // 4 + 64,
                                  dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] model ready in {time.time() - t0:.1f}s; "
            f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    def plan(self, n, r_p, r_kv, window=WINDOW):
        """(policy, T_sel, splits); window=n gives the KV-window baseline."""
        bc = self.bc
        pol = bc.policy(r_kv, SINKS, window)
        t_sel = bc.bc_kv_budget(n, pol)["t_sel"]
        S = bc.bc_attn_default_splits(t_sel, DIMS["n_kv_heads"])
        return pol, t_sel, S

    def step(self, n, r_p, r_kv, window=WINDOW, masked=False):
        bc = self.bc
        pol, _, S = self.plan(n, r_p, r_kv, window)
        if masked and self.masked_ws is None:
            D = DIMS
            self.masked_ws = torch.empty(bc.bc_masked_attn_workspace_bytes(self.max_ctx, D["n_heads"], D["head_dim"])
                                         // 4 + 64, dtype=torch.int32, device="cuda")
        st = bc.make_step(n, r_p, pol, S, masked_ws=self.masked_ws if masked else None)
        self.h.copy_(self.h0)
        bc.bc_decode_step(self.md, self.layer_array, self.g_final, self.w_head, st, self.h, self.logits, self.token,
                          self.ws)

    def graph(self, n, r_p, r_kv, window=WINDOW, masked=False):
        self.step(n, r_p, r_kv, window, masked)          # eager once: validates arguments outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(n, r_p, r_kv, window, masked)
        torch.cuda.synchronize()
        return g

    def layer_graph(self, n, r_p, r_kv, window=WINDOW):
        """One bc_decode_layer call (layer 0, residual stored at the end), as a
        graph: the per-layer latency."""
        bc = self.bc
        pol, _, S = self.plan(n, r_p, r_kv, window)
        st = bc.make_step(n, r_p, pol, S)

        def one():
            self.h.copy_(self.h0)
            bc.bc_decode_layer(self.md, self.c_layers[0], st, self.h, self.ws)
        one()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one()
        torch.cuda.synchronize()
        return g

    def sel_prepare(self, n, r_kv):
        """Select once and gather (not timed; README FAQ: the KV branch
        selects once after prefill, in SnapKV's way): every layer scores
        the tokens of its pre-filled cache by the pooled attention of its
        observation window (bc_kv_snap_select) and copies the kept tokens
        (sinks, history, window -- the last one being position n-1) into its
        compact cache (bc_kv_compact).  Returns T_sel."""
        bc = self.bc
        D = DIMS
        pol = bc.policy(r_kv, SINKS, WINDOW)
        t_sel = bc.bc_kv_snap_t_sel(n, pol)
        idx = self.sel_idx.view(-1)[:D["n_kv_heads"] * t_sel].view(D["n_kv_heads"], t_sel)
        for ly, q, (kc, vc) in zip(self.layers, self.sel_q, self.sel_kv):
            bc.bc_kv_snap_select(q, ly["k"], n, D["n_heads"], D["n_kv_heads"], pol, idx, None, self.sel_ws,
                                 pool_kernel=POOL)
            bc.bc_kv_compact(ly["k"], ly["v"], idx, t_sel, kc, vc)
        torch.cuda.synchronize()
        return t_sel

    def step_sel(self, t_sel, r_p):
        """A decode step over the gathered selections: the dense step at
        context T_sel (the current token rewrites slot T_sel - 1)."""
        bc = self.bc
        pol, _, S = self.plan(t_sel, r_p, 1.0)
        st = bc.make_step(t_sel, r_p, pol, S)
        self.h.copy_(self.h0)
        bc.bc_decode_step(self.md, self.layer_array_sel, self.g_final, self.w_head, st, self.h, self.logits,
                          self.token, self.ws)

    def graph_sel(self, n, r_p, r_kv):
        t_sel = self.sel_prepare(n, r_kv)
        self.step_sel(t_sel, r_p)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step_sel(t_sel, r_p)
        torch.cuda.synchronize()
        return g


SETTLE_S = 1.0         # untimed replays before a process's first timed graph
_settled = False


def settle(g, seconds=SETTLE_S):
    """Replays g, untimed, for about `seconds`: a GPU that was idle takes a
    few hundred ms of sustained load to reach its steady clocks (without
    this, a process's first 30-step timing of the dense 128K step read 4-5%
    slower than the same graph timed after it, and the cells right after it
    were slow too), so the first timed measurement of a process waits for
    that; later ones follow back-to-back work."""
    global _settled
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()
    _settled = True


def time_graph(g, steps, warmup):
    if not _settled:
        settle(g)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_read_probe(model, nbytes=512 << 20, reps=10, pool=1 << 30):
    """The practical HBM read ceiling at one launch size: bc_stream_read (256
    work-groups, two 16-byte non-temporal loads in flight per lane) over
    nbytes, rotating over the nbytes-sized pieces of a pool of at least two
    pieces and 1 GiB (beyond the 256 MB MALL), timed with events on the
    stream it runs on.  Returns (us per launch, bytes)."""
    bc = model.bc
    count = max(2, pool // nbytes)
    whole = torch.ones(count * nbytes // 4, dtype=torch.int32, device="cuda")
    bufs = [whole[i * (nbytes // 4):(i + 1) * (nbytes // 4)] for i in range(count)]
    sink = torch.empty(256, dtype=torch.int32, device="cuda")
    for b in bufs:
        bc.bc_stream_read(b, sink)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rounds = max(1, reps * 2 // count)
    e0.record(s)
    for _ in range(rounds):
        for b in bufs:
            bc.bc_stream_read(b, sink)
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / (rounds * len(bufs))
    del bufs, whole
    return us, nbytes


def replay_us(one_pass, launches, reps):
    """Per-launch time of `one_pass` (a pass of `launches` library calls on
    the current stream), replayed `reps` times from one HIP graph: what the
    GPU spends per launch back to back, with no host launch cost in it.  The
    pass runs once eagerly first (argument checks outside capture)."""
    one_pass()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_pass()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / (reps * launches)
    del g
    return us


def stream_us(one_pass, launches, reps):
    """Per-launch time of `one_pass` (a pass of `launches` library calls)
    launched `reps` times from the host onto the current stream, after one
    untimed pass, timed with events on that stream."""
    one_pass()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        one_pass()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / (reps * launches)


def time_attention_kernel(model, n, reps=3, S=None):
    """Average duration of bc_splitk_attn_partial over the 32 layers' caches
    (one launch per layer, as in the step), timed with events on the stream
    the kernels are launched on.  Launched from the host: each launch outlasts
    the host's launch cost, and stream launches sit closer together than the
    nodes of a graph replay, so the time per launch stays close to the
    kernel's own duration in a kernel trace."""
    bc = model.bc
    D = DIMS
    H, Hkv, hd = D["n_heads"], D["n_kv_heads"], D["head_dim"]
    S = S or bc.bc_attn_default_splits(n, Hkv)
    q = torch.randn((H, hd), dtype=torch.bfloat16, device="cuda").view(torch.int16)
    m = torch.empty((H, S), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    o = torch.empty((H, S, hd), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(hd)

    def one_pass():
        for ly in model.layers:
            bc.bc_splitk_attn_partial(q, ly["k"], ly["v"], None, n, H, Hkv, S, scale, m, l, o)
    us = stream_us(one_pass, len(model.layers), reps)
    return us, attn_bytes(n, S, False), S


def time_attention_sparse(model, n, r_kv, reps=3, S=None):
    """bc_splitk_attn_partial over a scored selection (the list of a random
    query), one launch per layer."""
    bc = model.bc
    D = DIMS
    H, Hkv, hd = D["n_heads"], D["n_kv_heads"], D["head_dim"]
    pol = bc.policy(r_kv, SINKS, WINDOW)
    bud = bc.bc_kv_budget(n, pol)
    t_sel = bud["t_sel"]
    S = S or bc.bc_attn_default_splits(t_sel, Hkv)
    q = torch.randn((H, hd), dtype=torch.bfloat16, device="cuda").view(torch.int16)
    idx = torch.empty((Hkv, t_sel), dtype=torch.int32, device="cuda")
    ws = torch.empty(bc.bc_kv_score_select_workspace_bytes(n, Hkv, pol) // 4 + 64, dtype=torch.int32, device="cuda")
    bc.bc_kv_score_select(q, model.layers[0]["summ"], n, H, Hkv, hd, pol, idx, None, ws)
    m = torch.empty((H, S), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    o = torch.empty((H, S, hd), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(hd)

    def one_pass():
        for ly in model.layers:
            bc.bc_splitk_attn_partial(q, ly["k"], ly["v"], idx, t_sel, H, Hkv, S, scale, m, l, o)
    us = stream_us(one_pass, len(model.layers), reps)
    return us, attn_bytes(t_sel, S, True), S


def time_select(n, k, reps=50):
    """bc_select_channels on an activation-distributed input, replayed in a
    HIP graph (so host launch cost is not timed)."""
    from activation_kv_cache_amd import binding as bc
    from activation_kv_cache_amd import inputs as gen
    x = torch.from_numpy(gen.activation_bf16(3, f"selbench{n}", n).view(np.int16)).cuda()
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    bc.bc_select_channels(x, k, idx)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            bc.bc_select_channels(x, k, idx)
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / reps


def kernel_table(model, contexts, split_sweep=None):
    """Per-kernel achieved bandwidth of the hot kernels (one launch per layer,
    rotating over the 32 layers' buffers): attention launched from the host,
    each row beside the streaming-read probe at about its byte count; the
    selections and GEMVs (launches as short as the host's own launch cost)
    replayed from HIP graphs."""
    rows = []
    for S in split_sweep or []:
        for n in contexts:
            for r_kv in (1.0, 0.3):
                if r_kv >= 1:
                    us, b, _ = time_attention_kernel(model, n, S=S)
                else:
                    us, b, _ = time_attention_sparse(model, n, r_kv, S=S)
                rows.append({"kernel": f"attn r_kv={r_kv} S={S}", "context": n, "us": round(us, 2), "bytes": b,
                             "gbs": round(b / us / 1e3, 1), "splits": S})
    def with_probe(row):
        # the streaming-read probe over about the same bytes (the nearest
        # multiple of 4 MiB): what one launch of that size reaches at best, so
        # launch ramp and kernel loss separate
        pb = max(1, round(row["bytes"] / (4 << 20))) << 22
        p_us, _ = time_read_probe(model, pb)
        row["probe_gbs"] = round(pb / p_us / 1e3, 1)
        row["frac_of_probe"] = round(row["gbs"] / row["probe_gbs"], 4)
        return row
    for n in contexts:
        us, b, S = time_attention_kernel(model, n)
        rows.append(with_probe({"kernel": "attn_partial dense", "context": n, "us": round(us, 2), "bytes": b,
                                "gbs": round(b / us / 1e3, 1), "splits": S}))
        for r_kv in (0.3, 0.5):
            us, b, S = time_attention_sparse(model, n, r_kv)
            rows.append(with_probe({"kernel": f"attn_partial r_kv={r_kv}", "context": n, "us": round(us, 2),
                                    "bytes": b, "gbs": round(b / us / 1e3, 1), "splits": S}))
    for n, k in ((4096, 2048), (4096, 2867), (14336, 7168), (14336, 10035)):
        us = time_select(n, k)
        rows.append({"kernel": f"select n={n} k={k}", "us": round(us, 2), "bytes": 2 * n + 4 * k,
                     "gbs": round((2 * n + 4 * k) / us / 1e3, 1)})
    for which in ("w_qkv", "w_o", "w_gu", "w_down"):
        for r_p in (1.0, 0.7, 0.5):
            us, b, k = time_gemv_kernel(model, which, r_p)
            rows.append({"kernel": f"gemv {which} r_p={r_p}", "us": round(us, 2), "bytes": b,
                         "gbs": round(b / us / 1e3, 1), "k": k})
    for r in rows:
        pr = (f"; probe {r['probe_gbs']:.0f} GB/s ({100 * r['probe_gbs'] / HBM_PEAK_GBS:.1f}%), kernel at "
              f"{100 * r['frac_of_probe']:.1f}% of it") if "probe_gbs" in r else ""
        log(f"[kernels] {r['kernel']:26s} {r.get('context', ''):>7} {r['us']:9.2f} us {r['gbs']:8.1f} GB/s "
            f"({100 * r['gbs'] / HBM_PEAK_GBS:.1f}%){pr}")
    return rows


def time_gemv_kernel(model, which="w_gu", r_p=1.0, reps=3):
    """Average duration of one bc_sparse_gemv_tiled call (its GEMV and, with
    several chunks, its finish kernel) over the 32 layers' matrices (dense or
    top-k channels of a fixed input), replayed from a HIP graph."""
    bc = model.bc
    from activation_kv_cache_amd import inputs as gen
    d_in, d_out = model.shapes[which]
    k = channel_keep(r_p, d_in)
    x = torch.from_numpy(gen.activation_bf16(1, "gemvx", d_in).view(np.int16)).cuda()
    idx = None
    if r_p < 1:
        idx = torch.empty(k, dtype=torch.int32, device="cuda")
        bc.bc_select_channels(x, k, idx)
    y = torch.empty(d_out, dtype=torch.int16, device="cuda")
    ws = torch.empty(bc.bc_sparse_gemv_workspace_bytes(d_out, k) // 4 + 64, dtype=torch.int32, device="cuda")
    bc.bc_workspace_init(ws)

    def one_pass():
        for ly in model.layers:
            bc.bc_sparse_gemv_tiled(ly[which], d_in, d_out, x, idx, k, y, ws)
    us = replay_us(one_pass, len(model.layers), reps)
    return us, gemv_bytes(d_in, d_out, k, r_p < 1), k


def time_library_gemv(d_in=4096, d_out=28672, count=4, reps=5, seed=0):
    """The same dense GEMV through torch.matmul in bf16 (the vendor BLAS),
    over `count` row-major matrices in turn (together beyond the 256 MB
    MALL): a strength check of the dense baseline.  Returns us per call."""
    from activation_kv_cache_amd import inputs as gen
    mats = [gen.device_normal_bf16(seed, f"libgemv{i}", (d_in, d_out), 0.02).view(torch.bfloat16) for i in range(count)]
    x = gen.device_normal_bf16(seed, "libgemvx", (1, d_in), 1.0).view(torch.bfloat16)
    for w in mats:
        torch.matmul(x, w)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        for w in mats:
            torch.matmul(x, w)
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / (reps * count)
    del mats
    return us


def time_batch_gemv(model, batch, r_p=0.5, which="w_gu", reps=3, seed=0):
    """The gate|up GEMV of `batch` sequences read once for the union of their
    channel lists (bc_sparse_gemv_batch) against `batch` single-sequence
    GEMVs, each over the 32 layers' matrices in turn.  Sequence b's input is
    N(0, 1) with the batch's shared 1% outlier channels x10, and its list is
    its own top-k (bc_select_channels)."""
    bc = model.bc
    from activation_kv_cache_amd import inputs as gen
    d_in, d_out = model.shapes[which]
    k = channel_keep(r_p, d_in)
    pos = gen.outlier_positions(seed, "batchx", d_in)
    xs = []
    for b in range(batch):
        v = gen.rng(seed, f"batchx/{b}").standard_normal(size=d_in, dtype=np.float32)
        v[pos] *= np.float32(10.0)
        xs.append(gen.to_bf16_bits(v))
    x = torch.from_numpy(np.stack(xs).view(np.int16)).cuda()
    idx = torch.empty((batch, k), dtype=torch.int32, device="cuda")
    for b in range(batch):
        bc.bc_select_channels(x[b], k, idx[b])
    y = torch.empty((batch, d_out), dtype=torch.int16, device="cuda")
    nu = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(bc.bc_sparse_gemv_batch_workspace_bytes(d_in, d_out, k, batch) // 4 + 64, dtype=torch.int32,
                     device="cuda")
    ws1 = torch.empty(bc.bc_sparse_gemv_workspace_bytes(d_out, k) // 4 + 64, dtype=torch.int32, device="cuda")
    bc.bc_workspace_init(ws)
    bc.bc_workspace_init(ws1)

    # |U| once (its count kernel is not part of the timed GEMV)
    bc.bc_sparse_gemv_batch(model.layers[0][which], x, idx, k, y, ws, n_union=nu, d_in=d_in, d_out=d_out, tiled=True)

    def batched(ly):
        bc.bc_sparse_gemv_batch(ly[which], x, idx, k, y, ws, d_in=d_in, d_out=d_out, tiled=True)

    def singles(ly):
        for b in range(batch):
            bc.bc_sparse_gemv_tiled(ly[which], d_in, d_out, x[b], idx[b], k, y[b], ws1)

    s = torch.cuda.current_stream()
    out = {}
    for label, fn in (("batched", batched), ("singles", singles)):
        for ly in model.layers[:2]:
            fn(ly)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            for ly in model.layers:
                fn(ly)
        e1.record(s)
        torch.cuda.synchronize()
        out[label] = e0.elapsed_time(e1) * 1000.0 / (reps * len(model.layers))
    n_union = int(nu.item())
    b = batch_gemv_bytes(n_union, d_in, d_out, k, batch)
    return {"batch": batch, "k": k, "union": n_union, "union_keep": round(n_union / d_in, 4),
            "us": round(out["batched"], 2), "bytes": b, "gbs": round(b / out["batched"] / 1e3, 1),
            "frac": round(b / out["batched"] / 1e3 / HBM_PEAK_GBS, 4), "singles_us": round(out["singles"], 2),
            "speedup_vs_singles": round(out["singles"] / out["batched"], 3),
            "crossover_batch_k": {str(r): round(batch_crossover_k(n_union / d_in, r, batch), 2) for r in (0.3, 0.5)}}


BATCH_SWEEPS = {2: [4096 * i for i in range(1, 11)], 4: [1024, 2048, 3072, 4096, 6144, 8192, 10240]}


def batch_crossover(model, B, contexts, steps, warmup, blocks=2, r_p=0.5, r_kv=0.3, seed=3):
    """A batch of B sequences sharing the weights (README "Quick start" /
    "Usage": crossover_batch): whole batched decode steps (bc_decode_step_batch:
    32 layers, the projections read once for the union of the sequences'
    channel lists, each sequence's own cache) in three modes -- dense, the
    projection branch (r_p) and the rescored KV branch (r_kv) -- at every
    context, in `blocks` shuffled blocks.  The crossing of the two branches'
    speedups over the batched dense step is compared with crossover_batch at
    the union keep measured on layer 0's channel lists (its GEMVs weighted by
    their weight bytes)."""
    bc = model.bc
    from activation_kv_cache_amd import inputs as gen
    D = DIMS
    d, dff, H, Hkv, hd, L = D["d"], D["d_ff"], D["n_heads"], D["n_kv_heads"], D["head_dim"], D["n_layers"]
    n_cap = max(contexts)
    caches = []
    for li in range(L):
        row = []
        for b in range(B):
            k = gen.device_normal_bf16(seed, f"batch{b}/layer{li}/kcache", (Hkv, n_cap, hd), 1.0)
            v = gen.device_normal_bf16(seed, f"batch{b}/layer{li}/vcache", (Hkv, n_cap, hd), 1.0)
            summ = torch.empty((Hkv, n_cap // 16, hd, 2), dtype=torch.int16, device="cuda")
            bc.bc_build_kv_summary(k, n_cap, summ)
            row.append((k, v, summ))
        caches.append(row)
    lys = [bc.make_layer(model.layers[li]["w_qkv"], model.layers[li]["w_o"], model.layers[li]["w_gu"],
                         model.layers[li]["w_down"], model.g_attn, model.g_mlp, *caches[li][b])
           for li in range(L) for b in range(B)]
    arr = bc.make_layer_array(lys)
    h0 = torch.from_numpy(np.stack([gen.activation_bf16(seed, f"batchh/{b}", d) for b in range(B)])
                          .view(np.int16)).cuda()
    hid = torch.empty_like(h0)
    logits = torch.empty((B, D["vocab"]), dtype=torch.float32, device="cuda")
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(bc.bc_layer_batch_workspace_bytes(model.md, B, n_cap, 64) // 4 + 64, dtype=torch.int32,
                     device="cuda")
    bc.bc_workspace_init(ws)

    # union keep of each GEMV input on layer 0 (channel lists from the taps)
    n0 = contexts[0]
    k_d, k_ff = channel_keep(r_p, d), channel_keep(r_p, dff)
    taps = [{k: torch.empty(m, dtype=torch.int32, device="cuda") for k, m in
             (("idx_qkv", k_d), ("idx_o", k_d), ("idx_gu", k_d), ("idx_down", k_ff))} for _ in range(B)]
    tarr = bc.make_taps_array([bc.make_taps(**t) for t in taps])
    hid.copy_(h0)
    bc.bc_decode_layer_batch(model.md, bc.make_layer_array(lys[:B]), bc.make_step(n0, r_p, bc.policy(1.0)), hid, ws,
                             taps_array=tarr)
    torch.cuda.synchronize()
    kvd = Hkv * hd
    wbytes = {"idx_qkv": (d, d * (H * hd + 2 * kvd)), "idx_o": (H * hd, H * hd * d), "idx_gu": (d, d * 2 * dff),
              "idx_down": (dff, dff * d)}
    union = {}
    for key, (d_in, w) in wbytes.items():
        u = np.unique(np.concatenate([t[key].cpu().numpy() for t in taps]))
        union[key] = u.size / d_in
    u_eff = sum(union[k] * wbytes[k][1] for k in wbytes) / sum(w for _, w in wbytes.values())

    modes = {"dense": (1.0, 1.0), "proj": (r_p, 1.0), "kv": (1.0, r_kv)}

    def graph(n, rp, rk):
        st = bc.make_step(n, rp, bc.policy(rk, SINKS, WINDOW), 0)

        def run():
            hid.copy_(h0)
            bc.bc_decode_step_batch(model.md, arr, L, B, model.g_final, model.w_head, st, hid, logits, tok, ws)
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        torch.cuda.synchronize()
        return g

    rng = np.random.default_rng(seed)
    cells = [(m, n) for m in modes for n in contexts]
    t = {m: np.zeros((blocks, len(contexts))) for m in modes}
    for blk in range(blocks):
        for ci in rng.permutation(len(cells)):
            m, n = cells[ci]
            g = graph(n, *modes[m])
            t[m][blk, contexts.index(n)] = time_graph(g, steps, warmup) * 1000.0
            del g
    sp = {m: (t["dense"] / t[m]).mean(axis=0) for m in ("proj", "kv")}
    c = crossing_k(contexts, [float(x) for x in sp["proj"] - sp["kv"]])
    pred = batch_crossover_k(u_eff, r_kv, B)
    kv_per_token = 2 * 2 * L * kvd
    w_proj = 2 * L * (2 * d * d + 2 * d * kvd + 3 * d * dff)
    pred_ext = (1 - u_eff) * w_proj / ((1 - r_kv - 1.0 / 16) * B * kv_per_token) / 1024
    rec = {"batch": B, "r_p": r_p, "r_kv": r_kv, "contexts": contexts, "blocks": blocks,
           "union_keep": {k: round(v, 4) for k, v in union.items()}, "union_keep_weighted": round(u_eff, 4),
           "step_us": {m: [round(x, 1) for x in t[m].mean(axis=0)] for m in modes},
           "speedup": {m: [round(x, 4) for x in sp[m]] for m in sp},
           "measured_k": None if c is None else round(c, 2), "crossover_batch_k": round(pred, 2),
           "crossover_batch_ext_k": round(pred_ext, 2)}
    log(f"[bench] batch {B}: union keep {u_eff:.3f}; crossing of the projection (r_p {r_p}) and KV (r_kv {r_kv}) "
        f"branches {rec['measured_k']}K, crossover_batch {pred:.1f}K (with the scored summaries {pred_ext:.1f}K); "
        f"dense step {rec['step_us']['dense'][0]} us at {contexts[0]}")
    del caches, lys, arr, ws
    torch.cuda.empty_cache()
    return rec


def load_traffic(n):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 counter summary, or None when the kernel sources changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", "attn_partial_dense_131072_pmc.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("context") != n:
        return None
    return rec.get("traffic_bytes_per_launch")


def all_sources_hash():
    """Hash of the code of every library source (csrc/*), comments and white
    space left out."""
    import glob
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "activation_kv_cache_amd", "csrc", "*"))):
        h.update(code_text(f).encode())
    return h.hexdigest()[:16]


def load_step_bytes():
    """Whole-step HBM bytes per mode against the byte account, from the
    committed counter summary (profiles/decode_step_bytes_pmc.json), with a
    flag telling whether the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "decode_step_bytes_pmc.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    cur = rec.get("kernel_sources_hash") == all_sources_hash()
    modes = rec.get("modes", [])
    return {"source": "profiles/decode_step_bytes_pmc.json", "kernel_sources_unchanged": cur, "modes": modes,
            "summary": {f"{m['mode']}@{m['context']}": [m["measured_over_algorithmic"], m["measured_over_page_account"]]
                        for m in modes} if cur else None}


def masked_comparison(n, steps, warmup):
    """The KV-window cell against two dense baselines (README FAQ "A KV method
    reports a speedup above its byte bound", paper Section 4.4; the
    abstract's "about fivefold"): the dense step with split-K attention and
    the dense step with masked attention (bc_masked_attn), all three on one
    model whose cache holds exactly n tokens (the masked baseline scans the
    whole cache).  Returns the record and frees the model."""
    model = Model(max_ctx=n, seed=2)
    t = {}
    for key, (r_p, r_kv, win, masked) in {"dense_splitk": (1.0, 1.0, WINDOW, False),
                                          "dense_masked": (1.0, 1.0, WINDOW, True),
                                          "kv_window_0.3": (1.0, 0.3, n, False)}.items():
        g = model.graph(n, r_p, r_kv, win, masked)
        t[key] = time_graph(g, steps, warmup) * 1000.0
        del g
    del model
    torch.cuda.empty_cache()
    bound = byte_bound(n, 1.0, 0.3)
    rec = {"context": n, "cache_slots": n, "step_us": {k: round(v, 1) for k, v in t.items()},
           "window_speedup_vs_splitk": round(t["dense_splitk"] / t["kv_window_0.3"], 3),
           "window_speedup_vs_masked": round(t["dense_masked"] / t["kv_window_0.3"], 3),
           "inflation": round(t["dense_masked"] / t["dense_splitk"], 3), "byte_bound": round(bound, 4)}
    rec["summary"] = {k: rec[k] for k in ("window_speedup_vs_splitk", "window_speedup_vs_masked", "inflation",
                                          "byte_bound")}
    log(f"[bench] KV window (r_kv 0.3) at {n}: {rec['window_speedup_vs_splitk']}x the split-K dense step, "
        f"{rec['window_speedup_vs_masked']}x the masked-attention dense step (inflation {rec['inflation']}x; "
        f"byte bound {bound:.2f}x); steps {rec['step_us']}")
    return rec


# Composition of the projection branch with the select-once KV branch (the
# pages' sel modes), as the README's headline speedups at 128K (A100) and its
# 32K composition table (RTX A6000) quote them: (r_p, r_kv) per context
COMPOSED_GRID = {131072: ((0.7, 1.0), (0.5, 1.0), (1.0, 0.3), (1.0, 0.5), (0.7, 0.3), (0.5, 0.3), (0.5, 0.5)),
                 32768: ((1.0, 0.2), (0.7, 0.2), (0.6, 0.2), (0.5, 0.2))}
PAGE_COMPOSED = {"131072": "A100: 1.91x composed, 1.54x KV selection, 1.15x activation sparsity (keep ratios not "
                           "stated)",
                 "32768": "RTX A6000: 1.20x / 1.53x / 1.69x / 1.86x at 1.0/0.2, 0.7/0.2, 0.6/0.2, 0.5/0.2"}


def composed_once(model, steps, warmup, rounds=3):
    """Speedups over the dense step of the projection branch, the select-once
    KV branch (selection made once after the pre-filled cache, gathered,
    then read densely by the unchanged split-K kernel) and their composition,
    at the contexts and keep ratios of COMPOSED_GRID (README "What it does in
    one picture" and "Timing and quality on a GPU"; paper Table 4 for 32K).
    Each round times the dense step and every cell of the context once,
    paired: a speedup is the mean over rounds of dense / cell."""
    rec = {"rounds": rounds, "steps": steps, "pages": PAGE_COMPOSED, "contexts": {}}
    for n, grid in COMPOSED_GRID.items():
        if n > model.max_ctx:
            continue
        t = {"dense": []}
        for _ in range(rounds):
            g = model.graph(n, 1.0, 1.0)
            t["dense"].append(time_graph(g, steps, warmup) * 1000.0)
            del g
            for r_p, r_kv in grid:
                key = f"{r_p}/{r_kv}"
                g = model.graph_sel(n, r_p, r_kv) if r_kv < 1 else model.graph(n, r_p, 1.0)
                t.setdefault(key, []).append(time_graph(g, steps, warmup) * 1000.0)
                del g
        dense = np.array(t["dense"])
        cells = {}
        for r_p, r_kv in grid:
            key = f"{r_p}/{r_kv}"
            tk = snap_t_sel(n, r_kv)
            b = step_bytes(tk, r_p, 1.0, *kv_plan(tk, 1.0))
            sp = float(np.mean(dense / np.array(t[key])))
            cells[key] = {"r_p": r_p, "r_kv": r_kv, "t_sel": tk, "step_us": round(float(np.mean(t[key])), 1),
                          "speedup": round(sp, 4), "byte_bound": round(byte_bound(n, r_p, r_kv), 4),
                          "bytes": b}
            log(f"[bench] select-once composition at {n}: r_p {r_p}, r_kv {r_kv}: {sp:.3f}x dense "
                f"(byte bound {byte_bound(n, r_p, r_kv):.2f}x), {np.mean(t[key]):.1f} us/step")
        rec["contexts"][str(n)] = {"dense_us": round(float(dense.mean()), 1), "cells": cells}
    rec["summary"] = {n: {k: [c["speedup"], c["byte_bound"]] for k, c in v["cells"].items()}
                      for n, v in rec["contexts"].items()}
    return rec


def cpu_baseline(model, n):
    """The CPU oracle, as it stands, on one decoder layer of the dense step at
    context n (layer 0's weights and cache copied to the host)."""
    import oracle

    D = DIMS
    ly = model.layers[0]
    t0 = time.time()

    def h16(t):
        return t.cpu().numpy().view(np.uint16)

    d, dff = D["d"], D["d_ff"]

    def untile(flat, d_in, d_out):
        out = np.empty((d_in, d_out), np.uint16)
        off = 0
        for t in range(0, d_out, 128):
            w = min(128, d_out - t)
            out[:, t:t + w] = flat[off:off + d_in * w].reshape(d_in, w)
            off += d_in * w
        return out

    gu = untile(h16(ly["w_gu"]), d, 2 * dff)
    # undo the per-tile gate | up interleave for the oracle's separate matrices
    gate = np.empty((d, dff), np.uint16)
    up = np.empty((d, dff), np.uint16)
    for t in range((dff + 63) // 64):
        w = min(64, dff - 64 * t)
        gate[:, 64 * t:64 * t + w] = gu[:, 128 * t:128 * t + w]
        up[:, 64 * t:64 * t + w] = gu[:, 128 * t + w:128 * t + 2 * w]
    W = dict(qkv=untile(h16(ly["w_qkv"]), *model.shapes["w_qkv"]), o=untile(h16(ly["w_o"]), *model.shapes["w_o"]),
             gate=gate, up=up, down=untile(h16(ly["w_down"]), *model.shapes["w_down"]),
             g1=h16(model.g_attn), g2=h16(model.g_mlp))
    K = h16(ly["k"][:, :n])
    V = h16(ly["v"][:, :n])
    summ = h16(ly["summ"])
    h = h16(model.h0)
    dims = dict(d=d, d_ff=dff, n_heads=D["n_heads"], n_kv_heads=D["n_kv_heads"], head_dim=D["head_dim"])
    log(f"[bench] cpu baseline inputs on host in {time.time() - t0:.1f}s")
    S = 1
    reps, elapsed = 0, 0.0
    while elapsed < 10.0 and reps < 200:   # about 10 s of host work
        t1 = time.perf_counter()
        oracle.decode_layer(h, W, K.copy(), V.copy(), summ.copy(), n, dims, 1.0, 1.0, SINKS, WINDOW, S)
        elapsed += time.perf_counter() - t1
        reps += 1
    sample_bytes = layer_bytes(n, 1.0, 1.0, n, S)
    # the same layer once more on one thread (thread counts only split
    # independent outputs, so the result is the same)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.decode_layer(h, W, K.copy(), V.copy(), summ.copy(), n, dims, 1.0, 1.0, SINKS, WINDOW, S)
        one = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(threads)
    # the LM head once (final norm + 128256 x 4096 GEMV), for the whole step
    # extrapolated as 32 x this layer + the LM head
    w_head = untile(h16(model.w_head), d, D["vocab"])
    t1 = time.perf_counter()
    oracle.lm_head(h, h16(model.g_final), w_head)
    head_s = time.perf_counter() - t1
    del w_head
    step_s = D["n_layers"] * elapsed / reps + head_s
    log(f"[bench] cpu oracle: one layer {elapsed / reps:.2f}s on {threads} threads, {one:.2f}s on one; "
        f"LM head {head_s:.2f}s; whole step (extrapolated) {step_s:.1f}s")
    cpu_model = ""
    try:
        cpu_model = next(ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round(sample_bytes * reps / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model, "layer_s": round(elapsed / reps, 3),
            "single_thread": {"value": round(sample_bytes / one / 1e9, 4), "layer_s": round(one, 3)},
            "step_extrapolated": {"s": round(step_s, 2), "lm_head_s": round(head_s, 3),
                                  "gbs": round(step_bytes(n, 1.0, 1.0, n, 32) / step_s / 1e9, 4),
                                  "how": "32 x the timed layer + the LM head timed once"},
            "sample": f"one of the 32 decoder layers of the dense {n}-token step (weights "
                      f"{layer_bytes(0, 1.0, 1.0, 0, 1) / 1e6:.0f} MB + KV {4096 * n / 1e6:.0f} MB), fp64 oracle, "
                      f"{reps} run(s) in {elapsed:.1f}s; GB/s = that layer's algorithmic bytes / oracle time"}


# mode -> (r_p, r_kv, select once): kv modes rescore the history every step;
# sel modes select once (after the pre-filled context) and step densely over
# the gathered selection, as the README's timing harness does
SWEEP_MODES = {"dense": (1.0, 1.0, False), "proj0.7": (0.7, 1.0, False), "proj0.5": (0.5, 1.0, False),
               "kv0.3": (1.0, 0.3, False), "kv0.5": (1.0, 0.5, False), "sel0.3": (1.0, 0.3, True),
               "sel0.5": (1.0, 0.5, True), "both0.7/0.3": (0.7, 0.3, False), "both0.5/0.3": (0.5, 0.3, False),
               "both0.5/0.5": (0.5, 0.5, False)}
PAIRS = (("proj0.7", "kv0.3", 0.7, 0.3), ("proj0.5", "kv0.3", 0.5, 0.3), ("proj0.5", "kv0.5", 0.5, 0.5),
         ("proj0.7", "sel0.3", 0.7, 0.3), ("proj0.5", "sel0.3", 0.5, 0.3), ("proj0.5", "sel0.5", 0.5, 0.5))


GEMV_IN = {0: "list", 1: "norm", 2: "sel", 3: "norm_sum", 4: "attn"}
GEMV_OUT = {0: "partial", 1: "bf16", 2: "swiglu", 3: "argmax"}
ATTN_LIST = {0: "dense", 1: "idx", 2: "scores"}


def phase_clock_launch(launch, clk):
    """Summary of one recorded launch (bc_phase_clocks_launches entry) from
    its clock slice (int64 numpy, 16 entries per work-group; include/bc.h):
    span and start skew from the real-time counter (10 ns), per-phase times
    of the median work-group from the shader clock (converted with its rate
    against the real-time counter), the last work-group's end after the
    median one, and per-XCC mean work-group times."""
    kind, a, b, c, d, groups, off = launch
    t = clk[off: off + 16 * groups].reshape(groups, 16).astype(np.float64)
    r0, r1, c0, c13 = t[:, 0], t[:, 1], t[:, 2], t[:, 13]
    ok = (r1 > r0) & (c13 > c0)
    mhz = 100.0 * float(np.median((c13 - c0)[ok] / (r1 - r0)[ok]))

    def ph(i, j):
        sel = (t[:, i] > 0) & (t[:, j] > 0)
        return round(float(np.median(t[sel, j] - t[sel, i])) / mhz, 3) if sel.any() else None
    rec = {"span_us": round((r1.max() - r0.min()) * 0.01, 3), "skew_us": round((r0.max() - r0.min()) * 0.01, 3),
           "last_after_median_us": round((r1.max() - np.median(r1)) * 0.01, 3), "mhz": round(mhz),
           "start_r": float(r0.min()), "end_r": float(r1.max())}
    xcc = t[:, 14].astype(np.int64) & 0xF
    rec["xcc_wg_us"] = {int(x): round(float(((r1 - r0)[xcc == x]).mean()) * 0.01, 3) for x in np.unique(xcc)}
    if kind == 1:
        rec["kernel"] = (f"k_gemv {GEMV_IN.get(a & 255)}/{GEMV_OUT.get(a >> 8)} {b}x{c}"
                         + ("" if d == b else f" k={d}") + f" ({groups} work-groups)")
        rec["phases_us"] = {"inputs_arrived": ph(2, 3), "input_formed": ph(2, 4), "selected": ph(2, 10),
                            "prologue": ph(2, 11), "row_loop": ph(11, 12), "epilogue": ph(12, 13),
                            "total": ph(2, 13)}
        if rec["phases_us"]["selected"] is not None:
            rec["selection_us"] = {"clear_and_barrier": ph(3, 4), "histogram": ph(4, 5), "wave_totals": ph(5, 6),
                                   "bin": ph(6, 7), "low_digit": ph(7, 8), "rank_scan": ph(8, 9), "emit": ph(9, 10)}
    else:
        rec["kernel"] = (f"k_attn_partial q={'partial' if (a & 255) else 'global'} list={ATTN_LIST.get(a >> 8)} "
                         f"{b} tokens, {c} splits ({groups} work-groups)")
        rec["phases_us"] = {"prologue": ph(2, 3), "rows_first_wave": ph(3, 12), "rows_all_waves": ph(3, 5),
                            "merge": ph(5, 13), "total": ph(2, 13)}
    return rec


def phase_clock_summary(model, specs, reps=5):
    """Per-phase clocks of every GEMV and attention launch of one decode step
    per (mode, context) spec, from the instrumented build: the step is
    captured in a HIP graph while recording (each launch takes its clock
    slice), replayed `reps` times, and the last replay's clocks are read.
    Launches of the same kernel and shape are averaged over the layers."""
    bc = model.bc
    buf = torch.zeros(16 << 20, dtype=torch.int64, device="cuda")
    out = {}
    for mode, n in specs:
        r_p, r_kv, once = SWEEP_MODES[mode]
        if once:
            t_sel = model.sel_prepare(n, r_kv)
            run = lambda: model.step_sel(t_sel, r_p)
        else:
            run = lambda: model.step(n, r_p, r_kv)
        run()
        torch.cuda.synchronize()
        buf.zero_()
        torch.cuda.synchronize()
        bc.bc_phase_clocks_begin(buf)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        launches = bc.bc_phase_clocks_launches()
        bc.bc_phase_clocks_begin(None)
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        clk = buf.cpu().numpy()
        recs = [phase_clock_launch(l, clk) for l in launches]
        for i in range(1, len(recs)):
            recs[i]["since_previous_us"] = round((recs[i]["start_r"] - recs[i - 1]["end_r"]) * 0.01, 3)
        groups = {}
        for r in recs:
            groups.setdefault(r["kernel"], []).append(r)
        rows = []
        for name, rs in groups.items():
            row = {"kernel": name, "launches": len(rs), "mhz": round(float(np.mean([r["mhz"] for r in rs])))}
            for key in ("span_us", "skew_us", "last_after_median_us"):
                row[key] = round(float(np.mean([r[key] for r in rs])), 3)
            gaps = [r["since_previous_us"] for r in rs if "since_previous_us" in r]
            # from the previous clocked launch's end (kernels without clocks
            # in between, such as the split-K reduce, count into it)
            row["since_previous_us"] = round(float(np.mean(gaps)), 3) if gaps else None
            for key in ("phases_us", "selection_us"):
                if key in rs[0]:
                    row[key] = {k: (None if rs[0][key][k] is None else
                                    round(float(np.mean([r[key][k] for r in rs if r[key][k] is not None])), 3))
                                for k in rs[0][key]}
            xs = sorted({x for r in rs for x in r["xcc_wg_us"]})
            row["xcc_wg_us"] = {x: round(float(np.mean([r["xcc_wg_us"][x] for r in rs if x in r["xcc_wg_us"]])), 3)
                                for x in xs}
            rows.append(row)
            ph_ = row["phases_us"]
            log(f"[clocks] {mode}@{n} {name} x{len(rs)}: span {row['span_us']:.2f} us, " +
                ", ".join(f"{k} {v:.2f}" for k, v in ph_.items() if v is not None) +
                (f"; selection " + ", ".join(f"{k} {v:.2f}" for k, v in row["selection_us"].items() if v is not None)
                 if "selection_us" in row else "") +
                f"; last work-group {row['last_after_median_us']:.2f} us after the median")
        out[f"{mode}@{n}"] = rows
        del g
    return out


CALIB_CONTEXTS = [2048, 16384, 32768, 65536, 98304, 131072, 163840]
CALIB_MODES = ("dense", "proj0.7", "proj0.5", "kv0.3", "kv0.5", "sel0.3", "sel0.5")


def time_cells(model, cells, steps, warmup, rng):
    """Step time (us) of every (mode, context) cell, in a shuffled order."""
    out = {}
    for ci in rng.permutation(len(cells)):
        m, n = cells[ci]
        r_p, r_kv, once = SWEEP_MODES[m]
        g = model.graph_sel(n, r_p, r_kv) if once else model.graph(n, r_p, r_kv)
        out[(m, n)] = time_graph(g, steps, warmup) * 1000.0
        del g
    return out


def calibration_sweep(model, blocks, steps, warmup, seed=1, contexts=None):
    """The branches' own sweeps for the cost-aware prediction (README
    "Results", paper Table 2: each branch's kernel cost comes from sweeps
    other than the one whose crossing is predicted): dense and every
    single-branch mode at a few contexts,
    in blocks of their own, timed before and apart from the crossover
    blocks whose crossings the prediction is compared with.  Returns the
    mean step time per mode over the blocks, [contexts]."""
    contexts = contexts or [n for n in CALIB_CONTEXTS if n <= model.max_ctx]
    rng = np.random.default_rng(seed)
    cells = [(m, n) for m in CALIB_MODES for n in contexts]
    t = {m: np.zeros((blocks, len(contexts))) for m in CALIB_MODES}
    for b in range(blocks):
        got = time_cells(model, cells, steps, warmup, rng)
        for (m, n), us in got.items():
            t[m][b, contexts.index(n)] = us
    log(f"[bench] calibration sweep: {len(cells)} cells x {blocks} blocks")
    return contexts, {m: t[m].mean(axis=0) for m in CALIB_MODES}


def crossover_sweep(model, contexts, blocks, steps, warmup, seed=0, calib=None):
    """Every mode at every context, `blocks` times in a shuffled order; the
    speedups S = t_dense / t_mode are paired within a block (README
    "Reproduce the paper": paired blocks), averaged over blocks, and each (r_p, r_kv)
    pair's crossing of S_proj and S_kv is compared with the byte-account n*
    and with the cost-aware prediction fitted on the separate calibration
    sweep `calib` = (contexts, mean step times per mode)."""
    rng = np.random.default_rng(seed)
    cells = [(m, n) for m in SWEEP_MODES for n in contexts]
    t = {m: np.zeros((blocks, len(contexts))) for m in SWEEP_MODES}
    for b in range(blocks):
        tb = time.time()
        got = time_cells(model, cells, steps, warmup, rng)
        for (m, n), us in got.items():
            t[m][b, contexts.index(n)] = us
        log(f"[bench] crossover block {b + 1}/{blocks} done in {time.time() - tb:.0f}s")
    sp = {m: (t["dense"] / t[m]).mean(axis=0) for m in SWEEP_MODES}
    out = {"contexts": contexts, "blocks": blocks, "steps": steps,
           "step_us": {m: [round(x, 1) for x in t[m].mean(axis=0)] for m in SWEEP_MODES},
           "speedup": {m: [round(x, 4) for x in sp[m]] for m in SWEEP_MODES if m != "dense"}, "pairs": {}}
    if calib:
        out["calibration"] = {"contexts": calib[0], "step_us": {m: [round(x, 1) for x in v]
                                                                  for m, v in calib[1].items()}}
    keys = [(f"{r_p}/{r_kv}" + (" sel" if SWEEP_MODES[mk][2] else ""), mp, mk) for mp, mk, r_p, r_kv in PAIRS]
    sp_iv, cross_iv = resample_intervals(t, contexts, keys)
    out["speedup_interval"] = sp_iv
    out["resamples"] = int(blocks ** blocks)
    plan = lambda n, a, b: model.plan(n, a, b)[1:]   # noqa: E731
    for mp, mk, r_p, r_kv in PAIRS:
        once = SWEEP_MODES[mk][2]
        d_vals = [float(x) for x in (t["dense"] / t[mp] - t["dense"] / t[mk]).mean(axis=0)]
        c = crossing_k(contexts, d_vals)
        # the sel branch moves exactly Eq. 5's bytes; the kv branch also reads
        # the summaries it rescores every step (n*_ext)
        ns, nx = n_star_k(r_p, r_kv), n_star_k(r_p, r_kv, ext=not once)
        key = f"{r_p}/{r_kv}" + (" sel" if once else "")
        rec = {"kv_policy": "select once, gathered" if once else "rescored every step",
               "n_star_k": round(ns, 2), "n_star_ext_k": round(nx, 2),
               "measured_k": None if c is None else round(c, 2),
               "measured_minus_n_star_k": None if c is None else round(c - ns, 2),
               "measured_minus_n_star_ext_k": None if c is None else round(c - nx, 2),
               "measured_interval": cross_iv[key]}
        # in-sample: costs fitted on the very sweep whose crossing is measured
        mean_t = {m: t[m].mean(axis=0) for m in ("dense", mp, mk)}
        pin, bw, cp, ck = predicted_crossing_k(contexts, mean_t, mp, mk, plan=plan)
        rec["pred_in_sample_k"] = None if pin is None else round(pin, 2)
        rec["pred_in_sample_fit"] = {"bw_gbs": round(bw, 1), "cost_proj_us": round(cp, 1), "cost_kv_us": round(ck, 1)}
        pred = None
        if calib:
            cctx, ct = calib
            pred, bw, cp, ck = predicted_crossing_k(cctx, ct, mp, mk, plan=plan)
            rec["pred_fit"] = {"bw_gbs": round(bw, 1), "cost_proj_us": round(cp, 1), "cost_kv_us": round(ck, 1),
                               "from": "separate calibration sweep"}
        rec["pred_k"] = None if pred is None else round(pred, 2)
        rec["measured_minus_pred_k"] = None if (c is None or pred is None) else round(c - pred, 2)
        out["pairs"][key] = rec
        iv = cross_iv[key]
        iv_s = f"[{iv['lo_k']:.1f}, {iv['hi_k']:.1f}]K" if "lo_k" in iv else "none"
        log(f"[bench] crossing {key}: measured {c if c is None else round(c, 1)}K "
            f"(95% over {iv['resamples']} block resamples {iv_s}), n* {ns:.1f}K, "
            f"n*_ext {nx:.1f}K, cost-aware prediction (separate sweep) "
            f"{pred if pred is None else round(pred, 1)}K, in-sample {pin if pin is None else round(pin, 1)}K")
    return out


def _read_counters(path):
    """(dispatch id, kernel name, counter value) rows of a rocprofv3
    counter-collection CSV."""
    import csv
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            did = r.get("Dispatch_Id") or r.get("Dispatch_ID") or r.get("dispatch_id")
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or r.get("kernel_name") or ""
            val = r.get("Counter_Value") or r.get("counter_value")
            if did is None or val is None:
                continue
            rows.append((int(did), name, float(val)))
    return rows


def kernel_key(name):
    """A kernel's name without its namespace and argument list, with its
    template arguments (k_gemv<3, 0, 4>)."""
    name = name.replace("void ", "").replace("(anonymous namespace)::", "").replace("bc::", "")
    return name.split("(")[0].strip()[:48]


def _copy_factor(path, copy_bytes):
    """KiB a counter reads per byte of a plain copy, from the copy dispatches
    (rocclr copyBuffer) of a --calib-copy run (which also fills its source)."""
    vals = [v for _, k, v in _read_counters(path) if "copyBuffer" in k]
    assert vals, f"no copy dispatch in {path}"
    return float(np.mean(vals)) * 1024 / copy_bytes


def attn_pmc_summary(fetch_csv, write_csv, cfetch_csv, cwrite_csv, n="131072", copy_bytes="1073741824"):
    """HBM bytes per launch of the attention kernel from two counter runs of
    --attn-only (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled
    by what the same counter reads for a plain copy; set against the
    kernel's algorithmic bytes (K and V of n tokens plus the partials).  The
    record carries the hash of the kernel's code, so that the bench reports
    this traffic only while the kernel is the one counted."""
    n, copy_bytes = int(n), int(copy_bytes)
    cf, cw = _copy_factor(cfetch_csv, copy_bytes), _copy_factor(cwrite_csv, copy_bytes)

    def per_dispatch(path):
        vals = [v for _, k, v in _read_counters(path) if kernel_key(k).startswith("k_attn_partial")]
        assert vals, f"no attention dispatch in {path}"
        return float(np.mean(vals)), len(vals)

    (fk, nd), (wk, _) = per_dispatch(fetch_csv), per_dispatch(write_csv)
    _, S = kv_plan(n, 1.0)
    algo = attn_bytes(n, S, False)
    traffic = fk * 1024 / cf + wk * 1024 / cw
    D = DIMS
    return {"kernel": f"k_attn_partial<{D['head_dim']}, {D['n_heads'] // D['n_kv_heads']}> "
                      f"(bc_splitk_attn_partial), dense, head_dim {D['head_dim']}, {D['n_kv_heads']} KV heads, "
                      f"{S} splits",
            "context": n, "kernel_source_hash": kernel_source_hash(),
            "kernel_source_hash_of": "code of bc_attn.hip + bc_device.hpp without comments and white space "
                                     "(bench.code_text)",
            "fetch_size_kib_per_dispatch": round(fk, 3), "write_size_kib_per_dispatch": round(wk, 3),
            "dispatches_averaged": nd,
            "copy_calibration": {"bytes": copy_bytes, "fetch_factor": round(cf, 6), "write_factor": round(cw, 6)},
            "traffic_bytes_per_launch": int(round(traffic)), "algorithmic_bytes_per_launch": algo,
            "traffic_over_algorithmic": round(traffic / algo, 4)}


def step_pmc_summary(fetch_csv, write_csv, cfetch_csv, cwrite_csv, specs, copy_bytes):
    """HBM bytes of one decode step per mode, from two counter runs of
    --step-pmc (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled
    by what the same counter reads for a plain copy of copy_bytes bytes.
    The dispatches between a mode's two marker launches (k_stream_read,
    before and after its steps) are that mode's REPS steps.  Each step is compared with its
    algorithmic bytes (step_bytes) and with the README's byte account
    r_p W_proj + W_head + (kept tokens) x KV bytes per token (README
    "Overview"; "Usage", the byte account).  Returns one record per mode."""
    specs = [(m, int(n), int(r)) for m, n, r in (x.split(":") for x in specs.split("+"))]
    copy_bytes = int(copy_bytes)
    cf, cw = _copy_factor(cfetch_csv, copy_bytes), _copy_factor(cwrite_csv, copy_bytes)

    def segments(path, factor):
        rows = sorted(_read_counters(path))
        marks = [d for d, k, _ in rows if "k_stream_read" in k]
        assert len(marks) == 2 * len(specs), f"{path}: {len(marks)} markers for {len(specs)} modes"
        out = []
        for i, (mode, n, reps) in enumerate(specs):
            lo, hi = marks[2 * i], marks[2 * i + 1]
            tot, by = 0.0, {}
            for d, k, v in rows:
                if lo < d < hi:
                    b = v * 1024 / factor / reps
                    tot += b
                    key = kernel_key(k)
                    by[key] = by.get(key, 0.0) + b
            out.append((tot, by))
        return out

    fseg = segments(fetch_csv, cf)
    wseg = segments(write_csv, cw)
    D = DIMS
    kvd = D["n_kv_heads"] * D["head_dim"]
    w_proj = 2 * D["n_layers"] * (2 * D["d"] ** 2 + 2 * D["d"] * kvd + 3 * D["d"] * D["d_ff"])
    w_head = 2 * D["vocab"] * D["d"]
    kv_tok = 2 * 2 * D["n_layers"] * kvd
    recs = []
    for (mode, n, reps), (fetch, fby), (write, wby) in zip(specs, fseg, wseg):
        r_p, r_kv, once = SWEEP_MODES[mode]
        t_sel, S = (snap_t_sel(n, r_kv), 0) if once else kv_plan(n, r_kv)
        algo = step_bytes(t_sel, r_p, 1.0, *kv_plan(t_sel, 1.0)) if once else step_bytes(n, r_p, r_kv, t_sel, S)
        kept = t_sel if r_kv < 1 else n
        account = r_p * w_proj + w_head + kept * kv_tok
        meas = fetch + write
        recs.append({"mode": mode, "context": n, "reps": reps, "t_sel": kept,
                     "fetch_bytes": round(fetch), "write_bytes": round(write), "measured_bytes": round(meas),
                     "algorithmic_bytes": algo, "page_account_bytes": round(account),
                     "measured_over_algorithmic": round(meas / algo, 4),
                     "measured_over_page_account": round(meas / account, 4),
                     "copy_factors": {"fetch": round(cf, 6), "write": round(cw, 6)},
                     "fetch_by_kernel": {k: round(v) for k, v in sorted(fby.items(), key=lambda x: -x[1])},
                     "write_by_kernel": {k: round(v) for k, v in sorted(wby.items(), key=lambda x: -x[1])}})
    return recs


def step_trace_summary(trace_csv, specs):
    """Per-mode kernel times of a rocprofv3 kernel trace of --step-pmc runs:
    after each mode's first marker launch, its REPS steps (each ending with
    the LM head's k_argmax_finish); the first two are left out as warm-up.
    Returns per mode the mean step time (first kernel start to last kernel
    end) and per kernel its launches per step and mean duration (us)."""
    import csv
    rows = []
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            rows.append((int(r["Dispatch_Id"]), kernel_key(r["Kernel_Name"]), int(r["Start_Timestamp"]),
                         int(r["End_Timestamp"])))
    rows.sort()
    specs = [(m, int(n), int(k)) for m, n, k in (x.split(":") for x in specs.split("+"))]
    marks = [i for i, r in enumerate(rows) if r[1].startswith("k_stream_read")]
    per = len(marks) // len(specs)
    out = []
    for si, (mode, n, reps) in enumerate(specs):
        steps, cur = [], []
        for r in rows[marks[si * per] + 1:]:
            cur.append(r)
            if r[1].startswith("k_argmax_finish"):
                steps.append(cur)
                cur = []
                if len(steps) == reps:
                    break
        use = steps[2:]
        wall = float(np.mean([st[-1][3] - st[0][2] for st in use])) / 1e3
        kern = {}
        for st in use:
            for _, k, a, b in st:
                e = kern.setdefault(k, [0, 0.0])
                e[0] += 1
                e[1] += (b - a) / 1e3
        ks = sorted(kern.items(), key=lambda kv: -kv[1][1])
        out.append({"mode": mode, "context": n, "steps": len(use), "step_us": round(wall, 1),
                    "launches_per_step": round(sum(v[0] for _, v in ks) / len(use), 1),
                    "kernels": [{"kernel": k, "per_step": round(v[0] / len(use), 1),
                                 "mean_us": round(v[1] / v[0], 2), "us_per_step": round(v[1] / len(use), 1)}
                                for k, v in ks]})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--contexts", default="2048,8192,32768,131072")
    ap.add_argument("--cells", default="default", help="default | dense | none | r_p:r_kv:n,...")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels", action="store_true", help="only the per-kernel bandwidth table")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="only copy this many bytes 5 times (calibration of the HBM byte counters)")
    ap.add_argument("--split-sweep", default="", help="attention split counts to sweep in --kernels")
    ap.add_argument("--crossover-blocks", type=int, default=5,
                    help="blocks of the crossover sweep (every mode at 2K, 4K, ..., 128K); 0 skips it")
    ap.add_argument("--crossover-steps", type=int, default=10, help="timed steps per sweep cell")
    ap.add_argument("--batch-sweep", type=int, default=1,
                    help="1: also time batched steps (2 and 4 sequences) and locate their crossing (0 skips it)")
    ap.add_argument("--calib-blocks", type=int, default=2,
                    help="blocks of the separate calibration sweep the cost-aware prediction is fitted on")
    ap.add_argument("--crossover-max-k", type=int, default=160,
                    help="largest context of the crossover sweep, in units of 1024 tokens (multiple of 4)")
    ap.add_argument("--gemv-only", default="",
                    help="reps:r_p -- only launch the gate|up GEMV reps times per layer (for counters)")
    ap.add_argument("--batch-only", type=int, default=0,
                    help="only the batched gate|up GEMV of this many sequences at r_p 0.5 (for counters)")
    ap.add_argument("--attn-only", type=int, default=0,
                    help="only launch the dense attention kernel this many times per layer (for counters)")
    ap.add_argument("--step-pmc", default="",
                    help="MODE:N:REPS[+MODE:N:REPS...] -- only REPS steps of each sweep mode at context N, each "
                         "mode's steps between two marker launches (bc_stream_read of 4 MiB), for whole-step "
                         "counters and kernel traces")
    ap.add_argument("--eager", action="store_true", help="with --step-pmc: eager steps instead of graph replays")
    ap.add_argument("--composed", action="store_true",
                    help="also time the select-once composition grid (part of the default run)")
    ap.add_argument("--phase-clocks", default="",
                    help="MODE:N+...: per-phase clocks of the GEMV and attention launches of one step per spec "
                         "(needs BC_LIBRARY=libbc_clk.so, the instrumented build)")
    ap.add_argument("--pmc-summary", default="",
                    help="FETCH_CSV,WRITE_CSV,CFETCH_CSV,CWRITE_CSV,SPECS,COPY_BYTES -- SPECS as for --step-pmc: "
                         "sum the counters of each mode's steps (between its two markers) and print each step's "
                         "HBM bytes against its byte account")
    ap.add_argument("--attn-pmc-summary", default="",
                    help="FETCH_CSV,WRITE_CSV,COPY_FETCH_CSV,COPY_WRITE_CSV[,N[,COPY_BYTES]] -- HBM bytes per "
                         "launch of the attention kernel from counter runs of --attn-only (the committed profile)")
    ap.add_argument("--trace-summary", default="",
                    help="TRACE_CSV,SPECS -- per-mode kernel times of a kernel trace of --step-pmc runs")
    ap.add_argument("--record", default=os.path.join(ROOT, "results", "bench_record.json"),
                    help="where the full record (cells, kernels, sweep) is written; the last stdout line is a "
                         "compact summary of it")
    args = ap.parse_args()

    if args.pmc_summary:
        recs = step_pmc_summary(*args.pmc_summary.split(","))
        # the committed profile: the records, the copy factors and the hash
        # of the library's code they were taken on
        print(json.dumps({"what": "HBM bytes of one whole decode step per mode (Llama-3.1-8B dims, 32 layers + "
                                  "LM head), eager steps, from two rocprofv3 counter passes scaled by a 1 GiB copy",
                          "copy_factors": recs[0]["copy_factors"] if recs else None,
                          "modes": recs, "kernel_sources_hash": all_sources_hash(),
                          "kernel_sources": "activation_kv_cache_amd/csrc/* (code without comments and white space)"},
                         indent=1))
        return
    if args.attn_pmc_summary:
        print(json.dumps(attn_pmc_summary(*args.attn_pmc_summary.split(",")), indent=1))
        return
    if args.trace_summary:
        print(json.dumps(step_trace_summary(*args.trace_summary.split(","))))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (no sharding or collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.calib_copy:
        src = torch.ones(args.calib_copy // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": src.numel() * 4}))
        return

    if args.phase_clocks:
        specs = [(m, int(n)) for m, n in (x.split(":") for x in args.phase_clocks.split("+"))]
        model = Model(max_ctx=max(n for _, n in specs))
        res = phase_clock_summary(model, specs)
        print(json.dumps({"phase_clocks": res, "library": model.bc.LIB_NAME}, separators=(",", ":")))
        return

    if args.step_pmc:
        specs = [(m, int(n), int(r)) for m, n, r in (x.split(":") for x in args.step_pmc.split("+"))]
        model = Model(max_ctx=max(n for _, n, _ in specs))
        sink = torch.empty(256, dtype=torch.int32, device="cuda")
        marker = torch.ones(1 << 20, dtype=torch.int32, device="cuda")
        for mode, n, reps in specs:
            r_p, r_kv, once = SWEEP_MODES[mode]
            t_sel = model.sel_prepare(n, r_kv) if once else None
            if args.eager:
                run = (lambda: model.step_sel(t_sel, r_p)) if once else (lambda: model.step(n, r_p, r_kv))
                run()
            else:
                g = model.graph_sel(n, r_p, r_kv) if once else model.graph(n, r_p, r_kv)
                run = g.replay
            torch.cuda.synchronize()
            model.bc.bc_stream_read(marker, sink)       # marks where this mode's steps begin
            for _ in range(reps):
                run()
            model.bc.bc_stream_read(marker, sink)       # and where they end
            torch.cuda.synchronize()
            log(f"[bench] steps only: {mode} at {n}: {reps} steps ({'eager' if args.eager else 'graph'})")
        print(json.dumps({"step_pmc": args.step_pmc}))
        return

    contexts = [int(c) for c in args.contexts.split(",")]
    head_n = max(contexts)
    sweep = (args.cells == "default" and args.crossover_blocks > 0 and head_n >= 131072 and not args.kernels
             and not args.attn_only and not args.gemv_only and not args.batch_only)
    # the crossover sweep runs past the headline context (to 160K tokens), so
    # that the 0.5/0.5 crossing (n*_ext 118.9K) is bracketed by measured cells
    sweep_ctx = [2048] + [4096 * i for i in range(1, args.crossover_max_k // 4 + 1)] if sweep else []
    model = Model(max_ctx=max(contexts + sweep_ctx))

    if args.kernels:
        sweep = [int(x) for x in args.split_sweep.split(",") if x]
        print(json.dumps({"kernels": kernel_table(model, contexts, sweep)}))
        return

    if args.gemv_only:
        reps, r_p = args.gemv_only.split(":")
        us, b, k = time_gemv_kernel(model, "w_gu", float(r_p), reps=int(reps))
        log(f"[bench] gate|up GEMV at r_p={r_p}: {us:.1f} us, {b / us / 1e3:.0f} GB/s, k={k}")
        print(json.dumps({"gemv_us": us, "gemv_bytes": b, "k": k}))
        return

    if args.batch_only:
        r = time_batch_gemv(model, args.batch_only, reps=1)
        log(f"[bench] batched gate|up GEMV, batch {args.batch_only}: {r['us']:.1f} us, union keep {r['union_keep']}")
        print(json.dumps({"batch_gemv": r}))
        return

    if args.attn_only:
        us, b, S = time_attention_kernel(model, head_n, reps=args.attn_only)
        log(f"[bench] attention kernel at n={head_n}: {us:.1f} us, {b / us / 1e3:.0f} GB/s, S={S}")
        print(json.dumps({"attn_us": us, "attn_bytes": b, "splits": S}))
        return

    # the dense step at each context (the headline is the largest); the
    # other modes are timed by the crossover sweep
    # a cell is (r_p, r_kv, n, kv policy): "scored" keeps sinks, the top
    # scored blocks and a 1024-token window; "window" is the KV-window
    # baseline (sinks and the most recent tokens, window = n)
    cells = [(1.0, 1.0, n, "scored") for n in contexts]
    if args.cells == "default":
        for n in sorted({min(contexts), head_n}):
            cells += [(0.5, 1.0, n, "scored"), (1.0, 0.3, n, "scored"), (0.5, 0.3, n, "scored"),
                      (1.0, 0.3, n, "window")]
    elif args.cells == "dense":
        pass
    elif args.cells == "none":
        cells = [(1.0, 1.0, head_n, "scored")]
    elif args.cells != "dense":
        # explicit list "r_p:r_kv:n[:window],..." (the dense cell at the largest context is always kept)
        cells = [(1.0, 1.0, head_n, "scored")] + [
            (float(f[0]), float(f[1]), int(f[2]), f[3] if len(f) > 3 else "scored")
            for f in (t.split(":") for t in args.cells.split(","))]

    results = []
    headline = None
    for (r_p, r_kv, n, kv) in cells:
        win = n if kv == "window" else WINDOW
        _, t_sel, S = model.plan(n, r_p, r_kv, win)
        g = model.graph(n, r_p, r_kv, win)
        is_head = (r_p, r_kv, n) == (1.0, 1.0, head_n)
        ms = time_graph(g, args.steps if is_head else min(args.steps, 20), args.warmup)
        del g
        b = step_bytes(n, r_p, r_kv, t_sel, S, kv != "window")
        gl = model.layer_graph(n, r_p, r_kv, win)
        lms = time_graph(gl, 50, args.warmup)
        del gl
        lb = layer_bytes(n, r_p, r_kv, t_sel, S, kv != "window")
        cell = {"r_p": r_p, "r_kv": r_kv, "context": n, "kv_policy": kv if r_kv < 1 else "dense",
                "step_us": round(ms * 1000, 1),
                "gbs": round(b / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "bytes": b, "t_sel": t_sel, "splits": S,
                "layer_us": round(lms * 1000, 2), "layer_bytes": lb,
                "layer_frac_hbm": round(lb / (lms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "byte_bound": round(byte_bound(n, r_p, r_kv), 4)}
        results.append(cell)
        log(f"[bench] r_p={r_p} r_kv={r_kv}{' (KV window)' if kv == 'window' and r_kv < 1 else ''} n={n}: "
            f"{cell['step_us']} us/step, {cell['gbs']} GB/s "
            f"({100 * cell['frac_hbm']:.1f}% of 8 TB/s); one layer {cell['layer_us']} us "
            f"({100 * cell['layer_frac_hbm']:.1f}%)")
        if is_head:
            headline = (ms, b)
    for c in results:
        dense = next((x for x in results if x["context"] == c["context"] and x["r_p"] == 1 and x["r_kv"] == 1), None)
        if dense:
            c["speedup_vs_dense"] = round(dense["step_us"] / c["step_us"], 3)
            if c is not dense:
                log(f"[bench] n={c['context']} r_p={c['r_p']} r_kv={c['r_kv']} {c['kv_policy']}: "
                    f"{c['speedup_vs_dense']}x dense (byte bound {c['byte_bound']:.2f}x)")

    ms, b = headline
    attn_us, attn_b, attn_S = time_attention_kernel(model, head_n)
    gemv_us, gemv_b, _ = time_gemv_kernel(model, "w_gu", 1.0)
    gemv_sp_us, gemv_sp_b, _ = time_gemv_kernel(model, "w_gu", 0.5)
    log(f"[bench] attention kernel {attn_us:.1f} us ({attn_b / attn_us / 1e3:.0f} GB/s); gate|up GEMV dense "
        f"{gemv_us:.1f} us ({gemv_b / gemv_us / 1e3:.0f} GB/s), r_p 0.5 {gemv_sp_us:.1f} us "
        f"({gemv_sp_b / gemv_sp_us / 1e3:.0f} GB/s)")
    achieved = attn_b / (attn_us * 1e-6) / 1e9
    probe_us, probe_b = time_read_probe(model)
    probe_gbs = probe_b / (probe_us * 1e-6) / 1e9
    log(f"[bench] streaming-read probe {probe_b >> 20} MiB: {probe_us:.1f} us ({probe_gbs:.0f} GB/s); attention at "
        f"{100 * achieved / probe_gbs:.0f}% of it")
    lib_us = time_library_gemv()
    log(f"[bench] the dense gate|up GEMV through torch.matmul (vendor BLAS, bf16): {lib_us:.1f} us "
        f"({gemv_b / lib_us / 1e3:.0f} GB/s); k_gemv {gemv_us:.1f} us")
    # the same probe at the gate|up GEMV's own sizes (224 and 112 MiB, within
    # 0.05% of its dense and r_p 0.5 bytes): a short launch pays its ramp too
    gemv_probe = {}
    for mib, (g_us, g_b) in ((224, (gemv_us, gemv_b)), (112, (gemv_sp_us, gemv_sp_b))):
        p_us, p_b = time_read_probe(model, mib << 20)
        p_gbs = p_b / p_us / 1e3
        gemv_probe[f"{mib}MiB"] = {"us": round(p_us, 2), "gbs": round(p_gbs, 1),
                                   "gemv_frac_of_probe": round(g_b / g_us / 1e3 / p_gbs, 4)}
        log(f"[bench] streaming-read probe {mib} MiB: {p_us:.1f} us ({p_gbs:.0f} GB/s); gate|up GEMV of that size at "
            f"{100 * g_b / g_us / 1e3 / p_gbs:.0f}% of it")
    out = {
        "metric": METRIC,
        "value": round(b / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: random-init N(0,0.02) weights of Llama-3.1-8B shape, N(0,1) pre-filled KV cache",
        "config": {"workload": f"dense decode step of one sequence at Llama-3.1-8B dims: 32 layers + LM head, "
                               f"context {head_n}, r_p=1, r_kv=1", "context": head_n, "r_p": 1.0, "r_kv": 1.0,
                   "layers": 32, "batch": 1},
        "roofline": {"bound": "hbm", "kernel": "k_attn_partial (bc_splitk_attn_partial), dense, one layer",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(head_n),
                     "launch_us": round(attn_us, 2), "bytes_per_launch": attn_b, "splits": attn_S},
        "read_probe": {"kernel": "bc_stream_read: 256 x 1024 lanes, two 16-byte non-temporal loads in flight per lane",
                       "bytes": probe_b, "us": round(probe_us, 2), "gbs": round(probe_gbs, 1),
                       "frac_of_peak": round(probe_gbs / HBM_PEAK_GBS, 4),
                       "attention_frac_of_probe": round(achieved / probe_gbs, 4)},
        "gemv_roofline": {"kernel": "k_gemv (bc_sparse_gemv), gate|up 4096x28672",
                          "dense": {"us": round(gemv_us, 2), "gbs": round(gemv_b / gemv_us / 1e3, 1),
                                    "frac": round(gemv_b / gemv_us / 1e3 / HBM_PEAK_GBS, 4)},
                          "r_p_0.5": {"us": round(gemv_sp_us, 2), "gbs": round(gemv_sp_b / gemv_sp_us / 1e3, 1),
                                      "frac": round(gemv_sp_b / gemv_sp_us / 1e3 / HBM_PEAK_GBS, 4)},
                          "read_probe_same_size": gemv_probe,
                          "vendor_blas_dense": {"us": round(lib_us, 2), "gbs": round(gemv_b / lib_us / 1e3, 1),
                                                "k_gemv_speedup": round(lib_us / gemv_us, 3),
                                                "how": "torch.matmul(x[1, 4096], W[4096, 28672]) in bf16"}},
        "cells": results,
    }
    out["step_bytes"] = load_step_bytes()
    # a batch of sequences through one union read of the gate|up weights
    out["batch_gemv"] = []
    for nb in (1, 2, 4):
        r = time_batch_gemv(model, nb)
        out["batch_gemv"].append(r)
        log(f"[bench] gate|up GEMV, batch {nb} at r_p 0.5: union keep {r['union_keep']:.3f}, {r['us']:.1f} us "
            f"({r['gbs']:.0f} GB/s, {100 * r['frac']:.1f}% of 8 TB/s) vs {r['singles_us']:.1f} us as {nb} single "
            f"GEMVs; batch crossover (r_kv 0.3) {r['crossover_batch_k']['0.3']:.1f}K")
    if args.cells == "default":
        out["kernels"] = kernel_table(model, contexts)
    if sweep:
        calib = calibration_sweep(model, args.calib_blocks, args.crossover_steps, min(args.warmup, 3))
        out["crossover"] = crossover_sweep(model, sweep_ctx, args.crossover_blocks, args.crossover_steps,
                                           min(args.warmup, 3), calib=calib)
    if sweep or args.composed:
        out["composed"] = composed_once(model, min(args.steps, 20), min(args.warmup, 3))
    if sweep and args.batch_sweep:
        out["batch_step"] = {"runs": [batch_crossover(model, B, BATCH_SWEEPS[B], args.crossover_steps,
                                                      min(args.warmup, 3)) for B in (2, 4)]}
        out["batch_step"]["summary"] = {f"b{r['batch']}": [r["measured_k"], r["crossover_batch_k"],
                                                          r["crossover_batch_ext_k"], r["union_keep_weighted"]]
                                        for r in out["batch_step"]["runs"]}
    if args.cells == "default" and head_n >= 131072:
        # on a model of its own (cache of exactly head_n slots), after the
        # headline cells
        out["masked_baseline"] = masked_comparison(head_n, min(args.steps, 10), args.warmup)
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(model, head_n)
        except Exception as e:  # the GPU figure stands on its own
            log(f"[bench] cpu baseline failed: {e!r}")
            out["cpu_baseline"] = None
    emit(out, args.record)


def emit(out, path):
    """Writes the full record to `path` (JSON) and prints the compact record
    as the last line of stdout."""
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        out["record_file"] = os.path.relpath(os.path.abspath(path), ROOT)
        with open(path, "w") as fh:
            json.dump(out, fh)
        log(f"[bench] full record written to {path}")
    print(compact_record(out), flush=True)


if __name__ == "__main__":
    main()
