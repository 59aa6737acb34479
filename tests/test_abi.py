"""The C ABI library loads and exports every entry point include/bc.h declares;
host-only queries agree with the oracle; argument errors are caught on the
host before anything is enqueued.  No device compute here (CPU suite)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bc.h")
LIB = os.path.join(ROOT, "activation_kv_cache_amd", "libbc.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bc_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def bc():
    if not os.path.exists(LIB):
        pytest.fail("libbc.so is not built: run __graft_entry__.build()")
    from activation_kv_cache_amd import binding
    return binding


def test_header_declares_the_six_calls():
    names = _declared()
    for n in ("bc_select_channels", "bc_sparse_gemv", "bc_kv_score_select", "bc_splitk_attn_partial",
              "bc_splitk_reduce", "bc_decode_layer"):
        assert n in names


def test_library_exports_every_declared_symbol(bc):
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared()) == set(bc.EXPORTED)


def test_abi_version(bc):
    assert bc.bc_abi_version() == 6


def test_phase_clocks_unsupported_in_the_library(bc):
    """The library itself records no phase clocks: its three clock entry
    points report BC_ERR_UNSUPPORTED (only libbc_clk.so, the instrumented
    build, records them)."""
    lib = bc.library()
    assert bc.LIB_NAME == "libbc.so"
    assert lib.bc_phase_clocks_begin(None, 0) == bc.BC_ERR_UNSUPPORTED
    assert lib.bc_phase_clocks_count() == bc.BC_ERR_UNSUPPORTED
    rec = (ctypes.c_longlong * 7)()
    assert lib.bc_phase_clocks_info(0, rec) == bc.BC_ERR_UNSUPPORTED
    with pytest.raises(bc.BcError):
        bc.bc_phase_clocks_begin(None)


@pytest.mark.parametrize("r_p,d", [(0.5, 4096), (0.7, 4096), (0.7, 14336), (0.5, 1408), (1.0, 77), (0.0001, 77),
                                   (0.25, 6), (0.3333, 1000)])
def test_channel_keep_matches_oracle(bc, r_p, d):
    assert bc.bc_channel_keep(r_p, d) == oracle.channel_keep(r_p, d)


@pytest.mark.parametrize("n,r_kv,sinks,window", [(2048, 0.3, 4, 128), (131072, 0.3, 4, 1024),
                                                 (131072, 0.5, 4, 1024), (2048, 0.3, 4, 1024),
                                                 (1999, 0.4, 4, 100), (5, 0.5, 4, 16), (1, 0.1, 4, 1024),
                                                 (4000, 1.0, 4, 1024), (3000, 0.0, 4, 16)])
def test_kv_budget_matches_oracle(bc, n, r_kv, sinks, window):
    got = bc.bc_kv_budget(n, bc.policy(r_kv, sinks, window))
    ref = oracle.kv_budget(n, r_kv, sinks, window)
    assert (got["t_sel"], got["k_blk"], got["n_cand"], got["b_lo"], got["sinks"], got["window"]) == (
        ref["T_sel"], ref["k_blk"], ref["n_cand"], ref["b_lo"], ref["sinks"], ref["window"])


def test_host_side_errors(bc):
    lib = bc.library()
    P = None
    # NULL pointers, bad sizes, unsupported head_dim, small workspace: all rejected before any launch
    assert lib.bc_select_channels(P, 10, 3, P, P) == bc.BC_ERR_INVALID
    assert lib.bc_select_channels(1 << 20, 10, 11, 1 << 20, P) == bc.BC_ERR_INVALID
    assert lib.bc_sparse_gemv(P, 10, 16, P, P, 10, P, P, 0, P) == bc.BC_ERR_INVALID
    assert lib.bc_sparse_gemv(1 << 20, 10, 12, 1 << 20, P, 10, 1 << 20, 1 << 20, 1 << 20, P) == bc.BC_ERR_UNSUPPORTED
    assert lib.bc_sparse_gemv(1 << 20, 64, 16, 1 << 20, P, 64, 1 << 20, 1 << 20, 1, P) == bc.BC_ERR_WORKSPACE
    assert lib.bc_splitk_attn_partial(1 << 20, 1 << 20, 1 << 20, 64, P, 64, 8, 2, 96, 1, 0.1, 1 << 20, 1 << 20,
                                      1 << 20, P) == bc.BC_ERR_UNSUPPORTED
    assert lib.bc_splitk_attn_partial(1 << 20, 1 << 20, 1 << 20, 64, P, 65, 8, 2, 64, 1, 0.1, 1 << 20, 1 << 20,
                                      1 << 20, P) == bc.BC_ERR_INVALID
    assert lib.bc_splitk_reduce(1 << 20, 1 << 20, 1 << 20, 8, 0, 64, 1 << 20, P) == bc.BC_ERR_INVALID
    # batched GEMV: NULL, batch outside [1, 4], d_in past the bitmaps, d_out % 8, k, workspace
    A = 1 << 20
    assert lib.bc_sparse_gemv_batch(P, 0, 64, 64, A, P, 64, 2, A, P, A, 1 << 30, P) == bc.BC_ERR_INVALID
    assert lib.bc_sparse_gemv_batch(A, 0, 64, 64, A, P, 64, 0, A, P, A, 1 << 30, P) == bc.BC_ERR_UNSUPPORTED
    assert lib.bc_sparse_gemv_batch(A, 0, 64, 64, A, P, 64, 5, A, P, A, 1 << 30, P) == bc.BC_ERR_UNSUPPORTED
    assert lib.bc_sparse_gemv_batch(A, 0, 16385, 64, A, P, 16385, 2, A, P, A, 1 << 30, P) == bc.BC_ERR_UNSUPPORTED
    assert lib.bc_sparse_gemv_batch(A, 0, 64, 60, A, P, 64, 2, A, P, A, 1 << 30, P) == bc.BC_ERR_UNSUPPORTED
    assert lib.bc_sparse_gemv_batch(A, 0, 64, 64, A, P, 32, 2, A, P, A, 1 << 30, P) == bc.BC_ERR_INVALID
    assert lib.bc_sparse_gemv_batch(A, 0, 64, 64, A, A, 65, 2, A, P, A, 1 << 30, P) == bc.BC_ERR_INVALID
    assert lib.bc_sparse_gemv_batch(A, 0, 64, 64, A, A, 16, 2, A, P, A, 16, P) == bc.BC_ERR_WORKSPACE
    assert bc.bc_sparse_gemv_batch_workspace_bytes(64, 64, 16, 5) == 0
    assert bc.bc_sparse_gemv_batch_workspace_bytes(4096, 28672, 2048, 4) > 0
    # the streaming-read probe: NULL, misaligned source, sizes that are not a positive multiple of 4 MiB
    assert lib.bc_stream_read(P, 4 << 20, 1 << 20, P) == bc.BC_ERR_INVALID
    assert lib.bc_stream_read((1 << 20) + 8, 4 << 20, 1 << 20, P) == bc.BC_ERR_INVALID
    assert lib.bc_stream_read(1 << 20, 0, 1 << 20, P) == bc.BC_ERR_INVALID
    assert lib.bc_stream_read(1 << 20, (4 << 20) + 16, 1 << 20, P) == bc.BC_ERR_INVALID
    pol = bc.policy(0.3, 4, 128, block=32)
    out = bc.bc_kv_budget_info()
    assert lib.bc_kv_budget(100, ctypes.byref(pol), ctypes.byref(out)) == bc.BC_ERR_UNSUPPORTED
    assert "block" in lib.bc_last_error().decode()
    md = bc.dims(dict(d=512, d_ff=1408, n_heads=8, n_kv_heads=2, head_dim=64))
    assert bc.bc_layer_workspace_bytes(md, 2048, 8) > 0
    bad = bc.dims(dict(d=500, d_ff=1408, n_heads=8, n_kv_heads=2, head_dim=64))
    assert bc.bc_layer_workspace_bytes(bad, 2048, 8) == 0


def test_noalloc_step_rejects_oversized_steps_on_the_host(bc):
    """bc_decode_step_noalloc checks the step's workspace against its static
    array before anything is enqueued (and before the array is looked up)."""
    lib = bc.library()
    md = bc.dims(dict(d=4096, d_ff=14336, n_heads=32, n_kv_heads=8, head_dim=128, vocab=128256, n_layers=1))
    A = 1 << 20
    n_cap = 600000
    ly = bc.bc_layer(A, A, A, A, A, A, A, A, A, n_cap)
    arr = bc.make_layer_array([ly])
    assert bc.bc_step_workspace_bytes(md, n_cap, bc.bc_attn_default_splits(n_cap, 8)) > bc.BC_STATIC_SCRATCH_BYTES
    st = bc.make_step(n_cap, 1.0, bc.policy(1.0))
    rc = lib.bc_decode_step_noalloc(ctypes.byref(md), arr, 1, A, A, ctypes.byref(st), A, A, A, None)
    assert rc == bc.BC_ERR_WORKSPACE
    assert "static" in lib.bc_last_error().decode()
    # NULL arguments are rejected the same way as by bc_decode_step
    rc = lib.bc_decode_step_noalloc(ctypes.byref(md), arr, 1, None, A, ctypes.byref(st), A, A, A, None)
    assert rc == bc.BC_ERR_INVALID


def test_workspace_queries_monotone(bc):
    md = bc.dims(dict(d=4096, d_ff=14336, n_heads=32, n_kv_heads=8, head_dim=128, vocab=128256))
    a = bc.bc_layer_workspace_bytes(md, 2048, 32)
    b = bc.bc_layer_workspace_bytes(md, 131072, 128)
    assert 0 < a < b < 64 << 20
    assert bc.bc_sparse_gemv_workspace_bytes(28672, 4096) >= bc.bc_sparse_gemv_workspace_bytes(28672, 2048) > 0
    assert bc.bc_lm_head_workspace_bytes(md) > 0


C_PROGRAM = r"""
#include <stdio.h>
#include "bc.h"

int main(void) {
  bc_kv_policy pol = {0.3, 4, 1024, 16};
  bc_kv_budget_info b;
  bc_model_dims md = {32, 4096, 14336, 128256, 32, 8, 128};
  if (bc_abi_version() != BC_ABI_VERSION) return 1;
  if (bc_channel_keep(0.5, 4096) != 2048) return 2;
  if (bc_kv_budget(131072, &pol, &b) != BC_OK || b.t_sel != 39316) return 3;
  if (bc_layer_workspace_bytes(&md, 131072, 32) == 0) return 4;
  if (bc_select_channels(NULL, 16, 4, NULL, NULL) != BC_ERR_INVALID) return 5;
  printf("%s\n", bc_last_error());
  return 0;
}
"""


def test_header_compiles_and_links_as_c(tmp_path):
    """include/bc.h is plain C: a C11 program includes it, links libbc.so and
    calls the host-only entry points (no device work)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(LIB):
        pytest.fail("libbc.so is not built: run __graft_entry__.build()")
    src = tmp_path / "abi.c"
    exe = tmp_path / "abi"
    src.write_text(C_PROGRAM)
    subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.dirname(HEADER), str(src), LIB,
                    "-Wl,-rpath," + os.path.dirname(LIB), "-o", str(exe)], check=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert "bc_select_channels" in run.stdout

