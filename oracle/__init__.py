"""CPU oracle of the decode step: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the bench's
cpu_baseline leg import this package.  It never imports the HIP library or
its binding, and the HIP library never imports it.

Source: "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
Decoding" (ByteCross), GitHub README page.  What each function follows:
  - byte account (byte_account.py): "Overview", "Quick start", "Usage",
    Table 1;
  - channel selection and sparse GEMV: "What it does in one picture" and
    "Timing and quality on a GPU" (activations select the projection weights
    read; all seven projections);
  - KV selection: "What it does in one picture" (sinks, part of the history,
    recent entries), scored per 16-token block by a key min/max bound; its
    gather into one contiguous buffer (the sel mode): "Timing and quality on
    a GPU";
  - the select-once policy in the SnapKV form (FAQ "How is this different
    from TEAL and SnapKV?"): observation-window attention votes, average
    pooling, per-head top-k of tokens;
  - split-K attention and its merge: "Overview" (one split-K attention kernel
    for every mode);
  - the layer: the Llama-3.1-8B decoder the README times (RMSNorm, rotary
    embedding, grouped-query attention, SwiGLU) -- its glue is not on the
    pages; eps 1e-5, rope theta 500000, unit norm gains are this oracle's
    choices and are parity unpinned.
Arithmetic: double everywhere, bf16 rounding where the step stores bf16;
block scores in float in one fixed order (see orc.c).

Arrays are numpy; bf16 tensors are uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

ROPE_THETA = 500000.0
RMS_EPS = 1e-5


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(HERE, "orc.c"))):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.orc_bf16_to_double.restype = D
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_from_double.restype = ctypes.c_uint16
    lib.orc_bf16_from_double.argtypes = [D]
    lib.orc_bf16_to_double_array.argtypes = [P, P, ctypes.c_long]
    lib.orc_bf16_from_double_array.argtypes = [P, P, ctypes.c_long]
    lib.orc_channel_keep.restype = I
    lib.orc_channel_keep.argtypes = [D, I]
    lib.orc_select_channels.argtypes = [P, I, I, P]
    lib.orc_sparse_gemv.argtypes = [P, I, I, P, P, I, P, P]
    lib.orc_rmsnorm.argtypes = [P, P, I, D, P]
    lib.orc_rope.argtypes = [P, I, I, I, D]
    lib.orc_swiglu.argtypes = [P, P, I, P]
    lib.orc_kv_summary.argtypes = [P, I, I, P]
    lib.orc_kv_budget.argtypes = [I, D, I, I, P]
    lib.orc_block_score.restype = ctypes.c_float
    lib.orc_block_score.argtypes = [P, P, I, I]
    lib.orc_kv_select.argtypes = [P, P, I, I, I, I, I, D, I, I, P, P]
    lib.orc_attn_partial.argtypes = [P, P, P, I, P, I, I, I, I, I, D, P, P, P]
    lib.orc_attn_reduce.argtypes = [P, P, P, I, I, I, P, P]
    lib.orc_snapkv_votes.argtypes = [P, P, I, I, I, I, I, I, D, P]
    lib.orc_avg_pool.argtypes = [P, I, I, P]
    lib.orc_token_budget.argtypes = [I, D, I, I, P]
    lib.orc_token_select.argtypes = [P, I, I, D, I, I, P]
    lib.orc_num_threads.restype = I
    lib.orc_set_num_threads.argtypes = [I]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- bf16 codec
def bf16_to_f64(a) -> np.ndarray:
    a = _c(a, np.uint16)
    out = np.empty(a.shape, np.float64)
    _load().orc_bf16_to_double_array(_p(a), _p(out), a.size)
    return out


def f64_to_bf16(a) -> np.ndarray:
    a = _c(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().orc_bf16_from_double_array(_p(a), _p(out), a.size)
    return out


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))


# ------------------------------------------------------- channel selection
def channel_keep(r_p: float, d_in: int) -> int:
    """k = floor(r_p * d_in + 1/2) clamped to [1, d_in]; r_p >= 1 -> d_in."""
    return _load().orc_channel_keep(float(r_p), int(d_in))


def select_channels(x, k: int) -> np.ndarray:
    """Top-k channels of |x| (ties: lower index), ascending int32."""
    x = _c(x, np.uint16)
    out = np.empty(k, np.int32)
    _load().orc_select_channels(_p(x), x.size, int(k), _p(out))
    return out


# ------------------------------------------------------------ sparse GEMV
def sparse_gemv(wt, x, idx=None, k=None):
    """y = W[:, S] x[S] with wt = W^T laid out [d_in][d_out].
    Returns (y64, y_bf16)."""
    wt = _c(wt, np.uint16)
    d_in, d_out = wt.shape
    x = _c(x, np.uint16)
    if idx is not None:
        idx = _c(idx, np.int32)
        k = idx.size
    elif k is None:
        k = d_in
    y64 = np.empty(d_out, np.float64)
    yb = np.empty(d_out, np.uint16)
    _load().orc_sparse_gemv(_p(wt), d_in, d_out, _p(x), _p(idx), int(k), _p(y64), _p(yb))
    return y64, yb


# ------------------------------------------------------------- layer glue
def rmsnorm(x, g, eps: float = RMS_EPS) -> np.ndarray:
    x = _c(x, np.uint16)
    g = _c(g, np.uint16)
    out = np.empty_like(x)
    _load().orc_rmsnorm(_p(x), _p(g), x.size, float(eps), _p(out))
    return out


def rope(v64, n_heads: int, head_dim: int, pos: int, theta: float = ROPE_THETA) -> np.ndarray:
    v = np.array(v64, dtype=np.float64, copy=True).reshape(-1)
    _load().orc_rope(_p(v), int(n_heads), int(head_dim), int(pos), float(theta))
    return v


def swiglu(gate64, up64) -> np.ndarray:
    gate64 = _c(gate64, np.float64)
    up64 = _c(up64, np.float64)
    out = np.empty(gate64.size, np.uint16)
    _load().orc_swiglu(_p(gate64), _p(up64), gate64.size, _p(out))
    return out


# ------------------------------------------------------------ KV selection
def kv_summary(k_head, n: int) -> np.ndarray:
    """Per-16-token-block (min, max) of one KV head's keys [n_cap][D]
    -> [ceil(n/16)][D][2] bf16."""
    k_head = _c(k_head, np.uint16)
    D = k_head.shape[-1]
    nb = (n + 15) // 16
    out = np.zeros((nb, D, 2), np.uint16)
    _load().orc_kv_summary(_p(k_head), int(n), int(D), _p(out))
    return out


def kv_budget(n: int, r_kv: float, sinks: int, window: int) -> dict:
    out = np.zeros(6, np.int32)
    _load().orc_kv_budget(int(n), float(r_kv), int(sinks), int(window), _p(out))
    keys = ("T_sel", "k_blk", "n_cand", "b_lo", "sinks", "window")
    return {k: int(v) for k, v in zip(keys, out)}


def block_score(q_group, summ_block) -> float:
    q_group = _c(q_group, np.uint16)
    summ_block = _c(summ_block, np.uint16)
    G, D = q_group.shape
    return float(_load().orc_block_score(_p(q_group), _p(summ_block), int(G), int(D)))


def kv_select(q, summ, n: int, n_heads: int, n_kv_heads: int, r_kv: float,
              sinks: int, window: int, want_scores: bool = False):
    """q [H][D] bf16; summ [Hkv][nb_cap][D][2] bf16 -> idx [Hkv][T_sel]
    (and scores [Hkv][n_cand] float32 when asked)."""
    q = _c(q, np.uint16)
    summ = _c(summ, np.uint16)
    D = q.shape[-1]
    nb_cap = summ.shape[1]
    bud = kv_budget(n, r_kv, sinks, window)
    idx = np.empty((n_kv_heads, bud["T_sel"]), np.int32)
    scores = np.empty((n_kv_heads, max(bud["n_cand"], 1)), np.float32) if want_scores else None
    _load().orc_kv_select(_p(q), _p(summ), int(nb_cap), int(n), int(n_heads), int(n_kv_heads),
                          int(D), float(r_kv), int(sinks), int(window), _p(idx), _p(scores))
    if want_scores:
        return idx, scores[:, :bud["n_cand"]]
    return idx


def kv_compact(K, V, idx, n_cap_out: int):
    """The scored selection copied into a buffer of its own, in list order (README
    "Timing and quality on a GPU": the sel mode; "API at a glance":
    select_and_compact): row t of head g of the output is row idx[g][t] of the
    cache.  K, V [Hkv][n_cap][D] bf16; idx [Hkv][T_sel] -> ([Hkv][n_cap_out][D]) x 2,
    rows past T_sel zero."""
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    idx = _c(idx, np.int32)
    Hkv, t_sel = idx.shape
    Ko = np.zeros((Hkv, n_cap_out, K.shape[2]), np.uint16)
    Vo = np.zeros_like(Ko)
    for g in range(Hkv):
        for t in range(t_sel):
            Ko[g, t] = K[g, idx[g, t]]
            Vo[g, t] = V[g, idx[g, t]]
    return Ko, Vo


# -------------------------------------------- select-once (SnapKV form) policy
def snapkv_votes(q_obs, K, n: int, n_heads: int, n_kv_heads: int, scale: float | None = None):
    """Attention votes of the observation queries q_obs [w][H][D] (bf16,
    positions n-w .. n-1) for every token t < n: [Hkv][n] double."""
    q_obs = _c(q_obs, np.uint16)
    K = _c(K, np.uint16)
    w, H, D = q_obs.shape
    assert H == n_heads
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((n_kv_heads, n), np.float64)
    _load().orc_snapkv_votes(_p(q_obs), _p(K), int(K.shape[1]), int(n), int(w), int(n_heads), int(n_kv_heads),
                             int(D), float(scale), _p(out))
    return out


def avg_pool(v, ks: int = 5) -> np.ndarray:
    """Average pooling of each row over ks neighbouring tokens (zero outside)."""
    v = _c(v, np.float64)
    out = np.empty_like(v)
    rows = v.reshape(-1, v.shape[-1])
    o = out.reshape(-1, v.shape[-1])
    for r in range(rows.shape[0]):
        row = np.ascontiguousarray(rows[r])
        res = np.empty_like(row)
        _load().orc_avg_pool(_p(row), row.size, int(ks), _p(res))
        o[r] = res
    return out


def token_budget(n: int, r_kv: float, sinks: int, window: int) -> dict:
    out = np.zeros(4, np.int32)
    _load().orc_token_budget(int(n), float(r_kv), int(sinks), int(window), _p(out))
    return dict(zip(("T_sel", "k", "sinks", "window"), (int(x) for x in out)))


def token_select(scores32, n: int, r_kv: float, sinks: int, window: int) -> np.ndarray:
    """Per KV head: sinks, the k highest float32 scores among the history
    candidates (ties: lower token) and the window, ascending [Hkv][T_sel]."""
    scores32 = _c(scores32, np.float32)
    Hkv = scores32.shape[0]
    bud = token_budget(n, r_kv, sinks, window)
    out = np.empty((Hkv, bud["T_sel"]), np.int32)
    _load().orc_token_select(_p(scores32), int(n), int(Hkv), float(r_kv), int(sinks), int(window), _p(out))
    return out


def snapkv_select(q_obs, K, n: int, n_heads: int, n_kv_heads: int, r_kv: float, sinks: int, window: int,
                  ks: int = 5):
    """The select-once list: votes of the observation window, average-pooled
    over ks tokens, rounded to float32 (the precision the decision is taken
    in) and ranked.  Returns (idx [Hkv][T_sel], pooled double [Hkv][n])."""
    pooled = avg_pool(snapkv_votes(q_obs, K, n, n_heads, n_kv_heads), ks)
    return token_select(pooled.astype(np.float32), n, r_kv, sinks, window), pooled


# --------------------------------------------------------------- attention
def attn_partial(q, K, V, idx, n_sel: int, n_heads: int, n_kv_heads: int, n_splits: int,
                 scale: float | None = None):
    """Split-K partials (m, l, o) in double; K, V are [Hkv][n_cap][D]."""
    q = _c(q, np.uint16)
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    n_cap, D = K.shape[1], K.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if idx is not None:
        idx = _c(idx, np.int32)
    m = np.empty((n_heads, n_splits), np.float64)
    l = np.empty((n_heads, n_splits), np.float64)
    o = np.empty((n_heads, n_splits, D), np.float64)
    _load().orc_attn_partial(_p(q), _p(K), _p(V), int(n_cap), _p(idx), int(n_sel), int(n_heads),
                             int(n_kv_heads), int(D), int(n_splits), float(scale),
                             _p(m), _p(l), _p(o))
    return m, l, o


def attn_reduce(m, l, o):
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    o = _c(o, np.float64)
    H, S, D = o.shape
    out64 = np.empty((H, D), np.float64)
    out = np.empty((H, D), np.uint16)
    _load().orc_attn_reduce(_p(m), _p(l), _p(o), int(H), int(S), int(D), _p(out64), _p(out))
    return out64, out


# -------------------------------------------------------------- one layer
def decode_layer(h, W: dict, K, V, summ, n: int, dims: dict, r_p: float, r_kv: float,
                 sinks: int, window: int, n_splits: int, forced: dict | None = None):
    """One decoder layer of the decode step, in the order

        x1 = RMSNorm(h); S1 = top-k(x1); q,k,v = W_qkv[:, S1] x1[S1];
        rotary on q, k; append k, v at slot n-1; refresh that block's summary;
        L = KV selection (r_kv < 1) or 0..n-1; a = attention(q, K[L], V[L]);
        S2 = top-k(a); h1 = h + W_o[:, S2] a[S2];
        x2 = RMSNorm(h1); S3 = top-k(x2); f = SiLU(W_g x2) * (W_u x2) over S3;
        S4 = top-k(f); h2 = h1 + W_d[:, S4] f[S4].

    W holds W^T matrices: 'qkv' [d][H*D + 2*Hkv*D], 'o' [H*D][d], 'gate' and
    'up' [d][d_ff], 'down' [d_ff][d], and the norm gains 'g1', 'g2' [d].
    K, V [Hkv][n_cap][D] and summ [Hkv][nb_cap][D][2] are updated in place.
    `forced` (teacher forcing) may hold any stage input produced elsewhere:
    x1, idx_qkv, q, k, v, idx_kv, a, idx_o, h_mid, x2, idx_gu, hff, idx_down;
    a forced value replaces this oracle's own value of that stage from then on.
    Returns every stage's value (the oracle's own output of each stage computed
    from the inputs in effect)."""
    f = forced or {}
    d, H, Hkv, D, dff = dims["d"], dims["n_heads"], dims["n_kv_heads"], dims["head_dim"], dims["d_ff"]
    out = {}

    def use(name, own):
        out[name] = own
        return f[name] if name in f else own

    k_d = channel_keep(r_p, d)
    k_ff = channel_keep(r_p, dff)
    sparse = r_p < 1.0

    x1 = use("x1", rmsnorm(h, W["g1"]))
    idx_qkv = use("idx_qkv", select_channels(x1, k_d) if sparse else None)
    qkv64, _ = sparse_gemv(W["qkv"], x1, idx_qkv)
    q64 = rope(qkv64[:H * D], H, D, n - 1)
    k64 = rope(qkv64[H * D:H * D + Hkv * D], Hkv, D, n - 1)
    v64 = qkv64[H * D + Hkv * D:]
    q = use("q", f64_to_bf16(q64).reshape(H, D))
    k = use("k", f64_to_bf16(k64).reshape(Hkv, D))
    v = use("v", f64_to_bf16(v64).reshape(Hkv, D))
    K[:, n - 1, :] = k
    V[:, n - 1, :] = v
    b = (n - 1) // 16
    for g in range(Hkv):
        summ[g, b] = kv_summary(K[g, 16 * b:n], n - 16 * b)[0]
    if r_kv < 1.0:
        idx_kv = use("idx_kv", kv_select(q, summ, n, H, Hkv, r_kv, sinks, window))
        n_sel = idx_kv.shape[1]
    else:
        idx_kv = use("idx_kv", None)
        n_sel = n
    m, l, o = attn_partial(q, K, V, idx_kv, n_sel, H, Hkv, n_splits)
    _, a = attn_reduce(m, l, o)
    a = use("a", a.reshape(H * D))
    idx_o = use("idx_o", select_channels(a, k_d) if sparse else None)
    yo64, _ = sparse_gemv(W["o"], a, idx_o)
    h_mid = use("h_mid", f64_to_bf16(bf16_to_f64(h) + yo64))
    x2 = use("x2", rmsnorm(h_mid, W["g2"]))
    idx_gu = use("idx_gu", select_channels(x2, k_d) if sparse else None)
    g64, _ = sparse_gemv(W["gate"], x2, idx_gu)
    u64, _ = sparse_gemv(W["up"], x2, idx_gu)
    hff = use("hff", swiglu(g64, u64))
    idx_down = use("idx_down", select_channels(hff, k_ff) if sparse else None)
    yd64, _ = sparse_gemv(W["down"], hff, idx_down)
    use("h_out", f64_to_bf16(bf16_to_f64(h_mid) + yd64))
    return out


def lm_head(h, g_final, w_head_t):
    """Final RMSNorm and the dense LM head: logits (double) and the argmax
    token (lowest index among equal maxima)."""
    x = rmsnorm(h, g_final)
    y64, _ = sparse_gemv(w_head_t, x)
    return x, y64, int(np.argmax(y64))
