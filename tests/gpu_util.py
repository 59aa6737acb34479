"""Helpers for the GPU parity tests: host <-> device copies of bf16 bit
patterns and the tolerance of the parity bar."""
import numpy as np
import torch

import oracle

ATOL, RTOL = 2e-3, 1e-2


def dev(a, device="cuda"):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to(device)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    raise TypeError(a.dtype)


def host_u16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


def empty_i16(n, device="cuda"):
    return torch.empty(n, dtype=torch.int16, device=device)


def workspace(nbytes, device="cuda"):
    from activation_kv_cache_amd import binding as bc
    ws = torch.empty(max(int(nbytes), 256) // 4 + 64, dtype=torch.int32, device=device)
    bc.bc_workspace_init(ws)
    return ws


def assert_close_bf16(got_u16, ref64, what="", atol=ATOL, rtol=RTOL):
    g = oracle.bf16_to_f64(got_u16).reshape(-1)
    r = np.asarray(ref64, dtype=np.float64).reshape(-1)
    err = np.abs(g - r)
    bad = err > atol + rtol * np.abs(r)
    rel_l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside {atol} + {rtol}|ref|; "
                           f"max err {err.max():.3g}, rel-L2 {rel_l2:.3g}")
    return rel_l2


def assert_close(got, ref64, what="", atol=ATOL, rtol=RTOL):
    g = np.asarray(got, dtype=np.float64).reshape(-1)
    r = np.asarray(ref64, dtype=np.float64).reshape(-1)
    err = np.abs(g - r)
    bad = err > atol + rtol * np.abs(r)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside; max err {err.max():.3g}"
