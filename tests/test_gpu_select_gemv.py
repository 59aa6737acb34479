"""GPU parity of channel selection (bit-exact index sets) and the sparse
projection GEMV (within 2e-3 + 1e-2|ref|) against the CPU oracle, through the
C ABI."""
import numpy as np
import pytest
import torch

import oracle
from activation_kv_cache_amd import inputs as gen

from gpu_util import assert_close_bf16, dev, host, host_u16, workspace

pytestmark = pytest.mark.gpu


def _bc():
    from activation_kv_cache_amd import binding as bc
    return bc


SELECT_CASES = [
    # (name, n, k, kind)
    ("tiny-x", 512, 256, "normal"),
    ("tiny-ff", 1408, 704, "normal"),
    ("8b-0.7", 4096, 2867, "outlier"),
    ("8b-0.5", 4096, 2048, "outlier"),
    ("8b-ff-0.7", 14336, 10035, "outlier"),
    ("8b-ff-0.5", 14336, 7168, "outlier"),
    ("ladder-few-levels", 4096, 1500, "ladder3"),
    ("ladder-all-equal", 1000, 333, "ladder1"),
    ("k1", 777, 1, "normal"),
    ("k-n", 300, 300, "normal"),
    ("k-n-minus-1", 300, 299, "ladder2"),
    ("ragged-small", 5, 3, "normal"),
    ("max-n", 65536, 40000, "outlier"),
    # the edges of the register-key paths (4 and 16 keys per thread) and the
    # radix path above them
    ("regs4-edge", 4097, 2049, "ladder5"),
    ("regs16-edge", 16384, 8191, "ladder7"),
    ("radix-edge", 16385, 8192, "outlier"),
]


def _make_x(n, kind, seed):
    if kind == "normal":
        return gen.normal_bf16(seed, f"selx{n}", n)
    if kind == "outlier":
        return gen.activation_bf16(seed, f"selx{n}", n)
    levels = int(kind[len("ladder"):])
    return gen.tie_ladder_bf16(n, levels, seed, f"ladder{n}")


@pytest.mark.parametrize("name,n,k,kind", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_select_channels_bit_exact(name, n, k, kind):
    bc = _bc()
    x = _make_x(n, kind, 11)
    idx = torch.full((k,), -1, dtype=torch.int32, device="cuda")
    bc.bc_select_channels(dev(x), k, idx)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), oracle.select_channels(x, k)), name


def test_select_signed_zero_and_specials():
    bc = _bc()
    x = np.array([0x8000, 0x0000, 0x3F80, 0xBF80, 0x0001, 0x8001, 0x7F7F, 0xFF7F], np.uint16)
    for k in range(1, 9):
        idx = torch.full((k,), -1, dtype=torch.int32, device="cuda")
        bc.bc_select_channels(dev(x), k, idx)
        torch.cuda.synchronize()
        assert np.array_equal(host(idx), oracle.select_channels(x, k)), k


GEMV_CASES = [
    # (name, d_in, d_out, r_p)
    ("tiny-qkv-dense", 512, 768, 1.0),
    ("tiny-qkv-0.5", 512, 768, 0.5),
    ("tiny-gu-0.5", 512, 2816, 0.5),
    ("tiny-down-0.5", 1408, 512, 0.5),
    ("ragged-out", 300, 520, 0.37),
    ("single-row", 64, 8, 1.0 / 64),
    ("8b-qkv-0.7", 4096, 6144, 0.7),
    ("8b-o-0.5", 4096, 4096, 0.5),
    ("8b-gu-0.5", 4096, 28672, 0.5),
    ("8b-down-0.7", 14336, 4096, 0.7),
    ("8b-down-dense", 14336, 4096, 1.0),
]


@pytest.mark.parametrize("name,d_in,d_out,r_p", GEMV_CASES, ids=[c[0] for c in GEMV_CASES])
def test_sparse_gemv_vs_oracle(name, d_in, d_out, r_p):
    bc = _bc()
    wt = gen.normal_bf16(5, f"gw{d_in}x{d_out}", (d_in, d_out), 0.02)
    x = gen.activation_bf16(5, f"gx{d_in}", d_in)
    k = oracle.channel_keep(r_p, d_in)
    dense = r_p >= 1.0
    idx_h = None if dense else oracle.select_channels(x, k)
    y = torch.empty(d_out, dtype=torch.int16, device="cuda")
    ws = workspace(bc.bc_sparse_gemv_workspace_bytes(d_out, k))
    bc.bc_sparse_gemv(dev(wt), dev(x), None if dense else dev(idx_h), k, y, ws)
    torch.cuda.synchronize()
    y64, _ = oracle.sparse_gemv(wt, x, idx_h, k)
    assert_close_bf16(host_u16(y), y64, name)
    # deterministic: a second call gives the same bits
    y2 = torch.empty_like(y)
    bc.bc_sparse_gemv(dev(wt), dev(x), None if dense else dev(idx_h), k, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_dense_gemv_equals_identity_list():
    """The same kernel serves both modes: idx = NULL and idx = 0..d_in-1 agree bit for bit."""
    bc = _bc()
    d_in, d_out = 4096, 4096
    wt = gen.normal_bf16(6, "gid", (d_in, d_out), 0.02)
    x = gen.activation_bf16(6, "gidx", d_in)
    ws = workspace(bc.bc_sparse_gemv_workspace_bytes(d_out, d_in))
    y1 = torch.empty(d_out, dtype=torch.int16, device="cuda")
    y2 = torch.empty(d_out, dtype=torch.int16, device="cuda")
    bc.bc_sparse_gemv(dev(wt), dev(x), None, d_in, y1, ws)
    bc.bc_sparse_gemv(dev(wt), dev(x), dev(np.arange(d_in, dtype=np.int32)), d_in, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_dense_gemv_vs_hipblaslt_strength():
    """A baseline-strength cross-check: the dense GEMV agrees with torch's
    bf16 matmul (hipBLASLt) in fp32 on the device."""
    bc = _bc()
    d_in, d_out = 4096, 6144
    wt = gen.device_normal_bf16(7, "gblas", (d_in, d_out), 0.02)
    x = gen.device_normal_bf16(7, "gblasx", (d_in,), 1.0)
    ws = workspace(bc.bc_sparse_gemv_workspace_bytes(d_out, d_in))
    y = torch.empty(d_out, dtype=torch.int16, device="cuda")
    bc.bc_sparse_gemv(wt, x, None, d_in, y, ws)
    ref = (x.view(torch.bfloat16).float() @ wt.view(torch.bfloat16).float())
    torch.cuda.synchronize()
    got = y.view(torch.bfloat16).float()
    assert torch.all((got - ref).abs() <= 2e-3 + 1e-2 * ref.abs())
