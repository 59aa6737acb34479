"""Thin Python binding of libbc (include/bc.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of the decode step; all of it runs in the HIP kernels.  torch
tensors provide device memory and the current stream.  If libbc.so is not
built, importing this module raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# BC_LIBRARY=libbc_clk.so selects the instrumented build (per-phase clocks;
# same kernels) from this directory; the default is the library itself
LIB_NAME = os.environ.get("BC_LIBRARY", "libbc.so")
if os.path.basename(LIB_NAME) != LIB_NAME or LIB_NAME not in ("libbc.so", "libbc_clk.so"):
    raise ImportError(f"BC_LIBRARY={LIB_NAME!r}: expected libbc.so or libbc_clk.so")
LIB_PATH = os.path.join(HERE, LIB_NAME)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_NAME} is not built ({LIB_PATH}); run __graft_entry__.build() first"
                      + (" and activation_kv_cache_amd/build.py --phase-clocks" if LIB_NAME != "libbc.so" else ""))

_lib = ctypes.CDLL(LIB_PATH)

c_int, c_double, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

BC_OK, BC_ERR_INVALID, BC_ERR_UNSUPPORTED, BC_ERR_WORKSPACE, BC_ERR_HIP = 0, -1, -2, -3, -4


class BcError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _lib.bc_last_error().decode(errors="replace")
        super().__init__(f"{where} failed with code {code}: {msg}")
        self.code = code


class bc_model_dims(ctypes.Structure):
    _fields_ = [("n_layers", c_int), ("d", c_int), ("d_ff", c_int), ("vocab", c_int),
                ("n_heads", c_int), ("n_kv_heads", c_int), ("head_dim", c_int)]


class bc_kv_policy(ctypes.Structure):
    _fields_ = [("r_kv", c_double), ("sinks", c_int), ("window", c_int), ("block", c_int)]


class bc_kv_budget_info(ctypes.Structure):
    _fields_ = [("t_sel", c_int), ("k_blk", c_int), ("n_cand", c_int), ("b_lo", c_int),
                ("sinks", c_int), ("window", c_int)]


class bc_layer(ctypes.Structure):
    _fields_ = [("w_qkv", c_void_p), ("w_o", c_void_p), ("w_gu", c_void_p), ("w_down", c_void_p),
                ("g_attn", c_void_p), ("g_mlp", c_void_p), ("k_cache", c_void_p), ("v_cache", c_void_p),
                ("kv_summary", c_void_p), ("n_cap", c_int)]


class bc_layer_taps(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("x1", "idx_qkv", "q", "k", "v", "idx_kv", "a", "idx_o", "h_mid", "x2",
                                        "idx_gu", "hff", "idx_down", "attn_m", "attn_l", "attn_o")]


class bc_step(ctypes.Structure):
    _fields_ = [("n_ctx", c_int), ("r_p", c_double), ("kv", bc_kv_policy), ("n_splits", c_int),
                ("rope_theta", c_double), ("rms_eps", c_double), ("taps", ctypes.POINTER(bc_layer_taps)),
                ("masked_ws", c_void_p), ("masked_ws_bytes", c_size_t)]


P = c_void_p
_SIG = {
    "bc_abi_version": (c_int, []),
    "bc_last_error": (ctypes.c_char_p, []),
    "bc_channel_keep": (c_int, [c_double, c_int]),
    "bc_kv_budget": (c_int, [c_int, ctypes.POINTER(bc_kv_policy), ctypes.POINTER(bc_kv_budget_info)]),
    "bc_workspace_init": (c_int, [P, c_size_t, P]),
    "bc_stream_read": (c_int, [P, c_size_t, P, P]),
    "bc_select_channels": (c_int, [P, c_int, c_int, P, P]),
    "bc_sparse_gemv_workspace_bytes": (c_size_t, [c_int, c_int]),
    "bc_sparse_gemv": (c_int, [P, c_int, c_int, P, P, c_int, P, P, c_size_t, P]),
    "bc_sparse_gemv_tiled": (c_int, [P, c_int, c_int, P, P, c_int, P, P, c_size_t, P]),
    "bc_sparse_gemv_batch_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
    "bc_sparse_gemv_batch": (c_int, [P, c_int, c_int, c_int, P, P, c_int, c_int, P, P, P, c_size_t, P]),
    "bc_kv_score_select_workspace_bytes": (c_size_t, [c_int, c_int, ctypes.POINTER(bc_kv_policy)]),
    "bc_kv_score_select": (c_int, [P, P, c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(bc_kv_policy), P, P,
                                   P, c_size_t, P]),
    "bc_build_kv_summary": (c_int, [P, c_int, c_int, c_int, c_int, P, P]),
    "bc_kv_compact": (c_int, [P, P, c_int, c_int, c_int, P, c_int, P, P, c_int, P]),
    "bc_kv_snap_t_sel": (c_int, [c_int, ctypes.POINTER(bc_kv_policy)]),
    "bc_kv_snap_select_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
    "bc_kv_snap_select": (c_int, [P, c_int, P, c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(bc_kv_policy), c_int,
                                  P, P, P, c_size_t, P]),
    "bc_splitk_attn_partial": (c_int, [P, P, P, c_int, P, c_int, c_int, c_int, c_int, c_int, c_float, P, P, P, P]),
    "bc_splitk_reduce": (c_int, [P, P, P, c_int, c_int, c_int, P, P]),
    "bc_attn_default_splits": (c_int, [c_int, c_int]),
    "bc_masked_attn_workspace_bytes": (c_size_t, [c_int, c_int, c_int]),
    "bc_masked_attn": (c_int, [P, P, P, c_int, c_int, c_int, c_int, c_int, c_float, P, P, c_size_t, P]),
    "bc_layer_workspace_bytes": (c_size_t, [ctypes.POINTER(bc_model_dims), c_int, c_int]),
    "bc_decode_layer": (c_int, [ctypes.POINTER(bc_model_dims), ctypes.POINTER(bc_layer), ctypes.POINTER(bc_step),
                                P, P, c_size_t, P]),
    "bc_pack_gate_up": (c_int, [P, P, c_int, c_int, P, P]),
    "bc_pack_weight_tiles": (c_int, [P, c_int, c_int, P, P]),
    "bc_lm_head_workspace_bytes": (c_size_t, [ctypes.POINTER(bc_model_dims)]),
    "bc_step_workspace_bytes": (c_size_t, [ctypes.POINTER(bc_model_dims), c_int, c_int]),
    "bc_decode_step": (c_int, [ctypes.POINTER(bc_model_dims), ctypes.POINTER(bc_layer), c_int, P, P,
                               ctypes.POINTER(bc_step), P, P, P, P, c_size_t, P]),
    "bc_decode_step_noalloc": (c_int, [ctypes.POINTER(bc_model_dims), ctypes.POINTER(bc_layer), c_int, P, P,
                                       ctypes.POINTER(bc_step), P, P, P, P]),
    "bc_layer_batch_workspace_bytes": (c_size_t, [ctypes.POINTER(bc_model_dims), c_int, c_int, c_int]),
    "bc_decode_layer_batch": (c_int, [ctypes.POINTER(bc_model_dims), ctypes.POINTER(bc_layer), c_int,
                                      ctypes.POINTER(bc_step), P, P, P, c_size_t, P]),
    "bc_decode_step_batch": (c_int, [ctypes.POINTER(bc_model_dims), ctypes.POINTER(bc_layer), c_int, c_int, P, P,
                                     ctypes.POINTER(bc_step), P, P, P, P, c_size_t, P]),
    "bc_lm_head": (c_int, [ctypes.POINTER(bc_model_dims), P, P, P, P, P, c_double, P, c_size_t, P]),
    "bc_phase_clocks_begin": (c_int, [P, c_size_t]),
    "bc_phase_clocks_count": (c_int, []),
    "bc_phase_clocks_info": (c_int, [c_int, ctypes.POINTER(ctypes.c_longlong)]),
}
for _name, (_res, _args) in _SIG.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIG)


def library():
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous CUDA/HIP tensors"
    return t.data_ptr()


def _stream(stream=None):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != BC_OK:
        raise BcError(rc, where)
    return rc


def _ws(t):
    return (_ptr(t), 0 if t is None else t.numel() * t.element_size())


def dims(d: dict) -> bc_model_dims:
    return bc_model_dims(d.get("n_layers", 1), d["d"], d["d_ff"], d.get("vocab", 8), d["n_heads"],
                         d["n_kv_heads"], d["head_dim"])


def policy(r_kv: float, sinks: int = 4, window: int = 1024, block: int = 16) -> bc_kv_policy:
    return bc_kv_policy(float(r_kv), int(sinks), int(window), int(block))


# ----------------------------------------------------------- host queries
def bc_abi_version() -> int:
    return _lib.bc_abi_version()


def bc_channel_keep(r_p: float, d_in: int) -> int:
    k = _lib.bc_channel_keep(float(r_p), int(d_in))
    if k < 0:
        raise BcError(k, "bc_channel_keep")
    return k


def bc_kv_budget(n_ctx: int, pol: bc_kv_policy) -> dict:
    out = bc_kv_budget_info()
    _check(_lib.bc_kv_budget(int(n_ctx), ctypes.byref(pol), ctypes.byref(out)), "bc_kv_budget")
    return {f: getattr(out, f) for f, _ in bc_kv_budget_info._fields_}


def bc_attn_default_splits(n_sel: int, n_kv_heads: int) -> int:
    return _lib.bc_attn_default_splits(int(n_sel), int(n_kv_heads))


def bc_sparse_gemv_workspace_bytes(d_out: int, k: int) -> int:
    return _lib.bc_sparse_gemv_workspace_bytes(int(d_out), int(k))


def bc_sparse_gemv_batch_workspace_bytes(d_in: int, d_out: int, k: int, batch: int) -> int:
    return _lib.bc_sparse_gemv_batch_workspace_bytes(int(d_in), int(d_out), int(k), int(batch))


def bc_kv_score_select_workspace_bytes(n_ctx: int, n_kv_heads: int, pol: bc_kv_policy) -> int:
    return _lib.bc_kv_score_select_workspace_bytes(int(n_ctx), int(n_kv_heads), ctypes.byref(pol))


def bc_layer_workspace_bytes(md: bc_model_dims, max_ctx: int, max_splits: int) -> int:
    return _lib.bc_layer_workspace_bytes(ctypes.byref(md), int(max_ctx), int(max_splits))


def bc_lm_head_workspace_bytes(md: bc_model_dims) -> int:
    return _lib.bc_lm_head_workspace_bytes(ctypes.byref(md))


# ------------------------------------------------------------ device calls
def bc_workspace_init(ws, stream=None):
    p, n = _ws(ws)
    return _check(_lib.bc_workspace_init(p, n, _stream(stream)), "bc_workspace_init")


def bc_phase_clocks_begin(buf=None):
    """Registers buf (an int64 device tensor) for the per-phase clocks of the
    launches that follow, or stops recording (None).  Raises BcError with
    BC_ERR_UNSUPPORTED unless the instrumented build is loaded."""
    if buf is None:
        return _check(_lib.bc_phase_clocks_begin(None, 0), "bc_phase_clocks_begin")
    return _check(_lib.bc_phase_clocks_begin(_ptr(buf), buf.numel() * buf.element_size()), "bc_phase_clocks_begin")


def bc_phase_clocks_launches():
    """The launches recorded since the last begin: a list of (kind, a, b, c,
    d, work-groups, first entry) tuples (include/bc.h)."""
    n = _lib.bc_phase_clocks_count()
    if n < 0:
        raise BcError(n, "bc_phase_clocks_count")
    out = []
    for i in range(n):
        rec = (ctypes.c_longlong * 7)()
        _check(_lib.bc_phase_clocks_info(i, rec), "bc_phase_clocks_info")
        out.append(tuple(int(v) for v in rec))
    return out


def bc_stream_read(src, sink, stream=None):
    """Measurement helper: one streaming read of the whole of src (its
    byte size a multiple of 4 MiB) into 256 checksum words at sink."""
    nbytes = src.numel() * src.element_size()
    return _check(_lib.bc_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "bc_stream_read")


def bc_select_channels(x, k: int, idx_out, stream=None):
    return _check(_lib.bc_select_channels(_ptr(x), x.numel(), int(k), _ptr(idx_out), _stream(stream)),
                  "bc_select_channels")


def bc_sparse_gemv(wt, x, idx, k: int, y, ws, stream=None):
    d_in, d_out = wt.shape
    p, n = _ws(ws)
    return _check(_lib.bc_sparse_gemv(_ptr(wt), d_in, d_out, _ptr(x), _ptr(idx), int(k), _ptr(y), p, n,
                                      _stream(stream)), "bc_sparse_gemv")


def bc_sparse_gemv_tiled(wt_packed, d_in: int, d_out: int, x, idx, k: int, y, ws, stream=None):
    p, n = _ws(ws)
    return _check(_lib.bc_sparse_gemv_tiled(_ptr(wt_packed), int(d_in), int(d_out), _ptr(x), _ptr(idx), int(k),
                                            _ptr(y), p, n, _stream(stream)), "bc_sparse_gemv_tiled")


def bc_sparse_gemv_batch(wt, x, idx, k: int, y, ws, n_union=None, d_in=None, d_out=None, tiled=False,
                         stream=None):
    """x [batch][d_in], idx [batch][k] or None, y [batch][d_out]; wt is
    [d_in][d_out] row-major, or tile-major (tiled=True: pass d_in, d_out)."""
    batch = x.shape[0]
    if not tiled:
        d_in, d_out = wt.shape
    p, n = _ws(ws)
    return _check(_lib.bc_sparse_gemv_batch(_ptr(wt), 1 if tiled else 0, int(d_in), int(d_out), _ptr(x), _ptr(idx),
                                            int(k), int(batch), _ptr(y), _ptr(n_union), p, n, _stream(stream)),
                  "bc_sparse_gemv_batch")


def bc_kv_score_select(q, summary, n_ctx: int, n_heads: int, n_kv_heads: int, head_dim: int,
                       pol: bc_kv_policy, idx_out, scores_out=None, ws=None, stream=None):
    nb_cap = summary.shape[1]
    p, n = _ws(ws)
    return _check(_lib.bc_kv_score_select(_ptr(q), _ptr(summary), nb_cap, int(n_ctx), int(n_heads), int(n_kv_heads),
                                          int(head_dim), ctypes.byref(pol), _ptr(idx_out), _ptr(scores_out), p, n,
                                          _stream(stream)), "bc_kv_score_select")


def bc_kv_snap_t_sel(n_ctx: int, pol: bc_kv_policy) -> int:
    t = _lib.bc_kv_snap_t_sel(int(n_ctx), ctypes.byref(pol))
    if t < 0:
        raise BcError(t, "bc_kv_snap_t_sel")
    return t


def bc_kv_snap_select_workspace_bytes(n_ctx: int, n_heads: int, n_kv_heads: int, w_obs: int) -> int:
    return _lib.bc_kv_snap_select_workspace_bytes(int(n_ctx), int(n_heads), int(n_kv_heads), int(w_obs))


def bc_kv_snap_select(q_obs, k_cache, n_ctx: int, n_heads: int, n_kv_heads: int, pol: bc_kv_policy, idx_out,
                      scores_out=None, ws=None, pool_kernel: int = 5, stream=None):
    """q_obs [w_obs][n_heads][head_dim], k_cache [n_kv_heads][n_cap][head_dim]."""
    w_obs, _, hd = q_obs.shape
    n_cap = k_cache.shape[1]
    p, n = _ws(ws)
    return _check(_lib.bc_kv_snap_select(_ptr(q_obs), int(w_obs), _ptr(k_cache), int(n_cap), int(n_ctx), int(n_heads),
                                         int(n_kv_heads), int(hd), ctypes.byref(pol), int(pool_kernel), _ptr(idx_out),
                                         _ptr(scores_out), p, n, _stream(stream)), "bc_kv_snap_select")


def bc_build_kv_summary(k_cache, n_ctx: int, summary, stream=None):
    n_kv, n_cap, hd = k_cache.shape
    return _check(_lib.bc_build_kv_summary(_ptr(k_cache), n_kv, n_cap, hd, int(n_ctx), _ptr(summary),
                                           _stream(stream)), "bc_build_kv_summary")


def bc_kv_compact(k_cache, v_cache, idx, t_sel: int, k_out, v_out, stream=None):
    n_kv, n_cap, hd = k_cache.shape
    return _check(_lib.bc_kv_compact(_ptr(k_cache), _ptr(v_cache), n_cap, n_kv, hd, _ptr(idx), int(t_sel),
                                     _ptr(k_out), _ptr(v_out), k_out.shape[1], _stream(stream)), "bc_kv_compact")


def bc_splitk_attn_partial(q, k_cache, v_cache, idx, n_sel: int, n_heads: int, n_kv_heads: int, n_splits: int,
                           scale: float, m, l, o, stream=None):
    _, n_cap, hd = k_cache.shape
    return _check(_lib.bc_splitk_attn_partial(_ptr(q), _ptr(k_cache), _ptr(v_cache), n_cap, _ptr(idx), int(n_sel),
                                              int(n_heads), int(n_kv_heads), hd, int(n_splits), float(scale),
                                              _ptr(m), _ptr(l), _ptr(o), _stream(stream)), "bc_splitk_attn_partial")


def bc_splitk_reduce(m, l, o, out, stream=None):
    n_heads, n_splits, hd = o.shape
    return _check(_lib.bc_splitk_reduce(_ptr(m), _ptr(l), _ptr(o), n_heads, n_splits, hd, _ptr(out),
                                        _stream(stream)), "bc_splitk_reduce")


def bc_masked_attn_workspace_bytes(n_cap: int, n_heads: int, head_dim: int) -> int:
    return _lib.bc_masked_attn_workspace_bytes(int(n_cap), int(n_heads), int(head_dim))


def bc_masked_attn(q, k_cache, v_cache, n_ctx: int, n_heads: int, n_kv_heads: int, scale: float, out, ws,
                   stream=None):
    _, n_cap, hd = k_cache.shape
    p, n = _ws(ws)
    return _check(_lib.bc_masked_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(n_cap), int(n_ctx), int(n_heads),
                                      int(n_kv_heads), int(hd), float(scale), _ptr(out), p, n, _stream(stream)),
                  "bc_masked_attn")


def bc_pack_gate_up(w_gate_t, w_up_t, w_gu, stream=None):
    d, d_ff = w_gate_t.shape
    assert w_gu.numel() == 2 * d * d_ff
    return _check(_lib.bc_pack_gate_up(_ptr(w_gate_t), _ptr(w_up_t), d, d_ff, _ptr(w_gu), _stream(stream)),
                  "bc_pack_gate_up")


def bc_pack_weight_tiles(wt, packed, stream=None):
    d_in, d_out = wt.shape
    return _check(_lib.bc_pack_weight_tiles(_ptr(wt), d_in, d_out, _ptr(packed), _stream(stream)),
                  "bc_pack_weight_tiles")


def packed_tiles(wt, stream=None):
    """A new device tensor holding wt in the tile-major layout."""
    out = torch.empty(wt.numel(), dtype=wt.dtype, device=wt.device)
    bc_pack_weight_tiles(wt, out, stream)
    return out


def make_layer(w_qkv, w_o, w_gu, w_down, g_attn, g_mlp, k_cache, v_cache, kv_summary=None) -> bc_layer:
    return bc_layer(_ptr(w_qkv), _ptr(w_o), _ptr(w_gu), _ptr(w_down), _ptr(g_attn), _ptr(g_mlp), _ptr(k_cache),
                    _ptr(v_cache), _ptr(kv_summary), int(k_cache.shape[1]))


def make_taps(**bufs) -> bc_layer_taps:
    return bc_layer_taps(**{k: _ptr(v) for k, v in bufs.items()})


def make_step(n_ctx: int, r_p: float, pol: bc_kv_policy, n_splits: int = 0, rope_theta: float = 500000.0,
              rms_eps: float = 1e-5, taps: bc_layer_taps | None = None, masked_ws=None) -> bc_step:
    """masked_ws: a device workspace for the masked-attention dense baseline
    (None: split-K attention)."""
    mp, mn = _ws(masked_ws)
    st = bc_step(int(n_ctx), float(r_p), pol, int(n_splits), float(rope_theta), float(rms_eps), None, mp, mn)
    if taps is not None:
        st.taps = ctypes.pointer(taps)
    return st


def bc_decode_layer(md: bc_model_dims, layer: bc_layer, step: bc_step, hidden, ws, stream=None):
    p, n = _ws(ws)
    return _check(_lib.bc_decode_layer(ctypes.byref(md), ctypes.byref(layer), ctypes.byref(step), _ptr(hidden), p,
                                       n, _stream(stream)), "bc_decode_layer")


def bc_lm_head(md: bc_model_dims, hidden, g_final, w_head_t, logits, token, rms_eps: float, ws, stream=None):
    p, n = _ws(ws)
    return _check(_lib.bc_lm_head(ctypes.byref(md), _ptr(hidden), _ptr(g_final), _ptr(w_head_t), _ptr(logits),
                                  _ptr(token), float(rms_eps), p, n, _stream(stream)), "bc_lm_head")


def bc_step_workspace_bytes(md: bc_model_dims, max_ctx: int, max_splits: int) -> int:
    return _lib.bc_step_workspace_bytes(ctypes.byref(md), int(max_ctx), int(max_splits))


def make_layer_array(layers):
    """A ctypes array of bc_layer structs (kept alive by the caller)."""
    arr = (bc_layer * len(layers))()
    for i, ly in enumerate(layers):
        arr[i] = ly
    return arr


def bc_decode_step(md: bc_model_dims, layer_array, g_final, w_head, step: bc_step, hidden, logits, token, ws,
                   stream=None):
    p, n = _ws(ws)
    return _check(_lib.bc_decode_step(ctypes.byref(md), layer_array, len(layer_array), _ptr(g_final), _ptr(w_head),
                                      ctypes.byref(step), _ptr(hidden), _ptr(logits), _ptr(token), p, n,
                                      _stream(stream)), "bc_decode_step")


BC_STATIC_SCRATCH_BYTES = 16 << 20


def bc_decode_step_noalloc(md: bc_model_dims, layer_array, g_final, w_head, step: bc_step, hidden, logits, token,
                           stream=None):
    """bc_decode_step with the library's static workspace (no ws argument)."""
    return _check(_lib.bc_decode_step_noalloc(ctypes.byref(md), layer_array, len(layer_array), _ptr(g_final),
                                              _ptr(w_head), ctypes.byref(step), _ptr(hidden), _ptr(logits),
                                              _ptr(token), _stream(stream)), "bc_decode_step_noalloc")


def bc_layer_batch_workspace_bytes(md: bc_model_dims, batch: int, max_ctx: int, max_splits: int) -> int:
    return _lib.bc_layer_batch_workspace_bytes(ctypes.byref(md), int(batch), int(max_ctx), int(max_splits))


def make_taps_array(taps):
    arr = (bc_layer_taps * len(taps))()
    for i, t in enumerate(taps):
        arr[i] = t
    return arr


def bc_decode_layer_batch(md: bc_model_dims, layer_array, step: bc_step, hidden, ws, taps_array=None, stream=None):
    """layer_array: bc_layer per sequence (shared weights, own caches);
    hidden [batch][d]."""
    p, n = _ws(ws)
    tp = ctypes.cast(taps_array, c_void_p) if taps_array is not None else None
    return _check(_lib.bc_decode_layer_batch(ctypes.byref(md), layer_array, len(layer_array), ctypes.byref(step),
                                             _ptr(hidden), tp, p, n, _stream(stream)), "bc_decode_layer_batch")


def bc_decode_step_batch(md: bc_model_dims, layer_array, n_layers: int, batch: int, g_final, w_head, step: bc_step,
                         hidden, logits, tokens, ws, stream=None):
    """layer_array: [n_layers * batch] bc_layer, layer-major."""
    p, n = _ws(ws)
    return _check(_lib.bc_decode_step_batch(ctypes.byref(md), layer_array, int(n_layers), int(batch), _ptr(g_final),
                                            _ptr(w_head), ctypes.byref(step), _ptr(hidden), _ptr(logits),
                                            _ptr(tokens), p, n, _stream(stream)), "bc_decode_step_batch")
