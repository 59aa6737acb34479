"""An order-independent check of a KV block selection.

The block score of KV head g and block b is, in real arithmetic, the sum
over the group's query heads j and the dims d of max(q_jd * kmax_bd,
q_jd * kmin_bd) -- an upper bound of q_j . k_t over the block's tokens (the
Quest form).  Computed here in float64 straight from that definition, with
numpy, independently of the oracle's and the kernel's fixed float32 order.

A float32 evaluation in any fixed order of at most 16 roundings along a
path differs from the exact value by at most
    band_b = 16 * 2^-24 * sum_j sum_d |max(q_jd kmax_bd, q_jd kmin_bd)|
(first-order bound of a sum of roundings, each relative error <= 2^-24;
the documented order has at most 12: up to 3 adds of the group's positive
or negative parts, one product, one fused multiply-add, two adds of a dim
group of 4 and 5 levels of the tree over 32 groups).  So the kept set is a
valid top-k of the float32 scores only if it is a top-k of the exact scores
up to swaps within those bands:
    min over kept b of (s_b + band_b) >= max over dropped c of (s_c - band_c).
"""
import numpy as np

BAND_ROUNDINGS = 16


def bf16_bits_to_f64(a):
    a = np.asarray(a, np.uint16).astype(np.uint32) << 16
    return a.view(np.float32).astype(np.float64)


def plain_scores(q, summ, n_cand, b_lo):
    """q [H][D] bf16 bits; summ [Hkv][nb][D][2] bf16 bits (min, max).
    Returns (scores, bands), each [Hkv][n_cand] float64."""
    H, D = q.shape
    Hkv = summ.shape[0]
    G = H // Hkv
    qf = bf16_bits_to_f64(q)
    s = np.zeros((Hkv, n_cand))
    band = np.zeros((Hkv, n_cand))
    for g in range(Hkv):
        blk = summ[g, b_lo:b_lo + n_cand]
        mn = bf16_bits_to_f64(blk[..., 0])           # [n_cand][D]
        mx = bf16_bits_to_f64(blk[..., 1])
        for j in range(g * G, (g + 1) * G):
            t = np.maximum(qf[j][None, :] * mx, qf[j][None, :] * mn)
            s[g] += t.sum(axis=1)
            band[g] += np.abs(t).sum(axis=1)
    return s, BAND_ROUNDINGS * 2.0 ** -24 * band


def kept_blocks(idx_g, sinks, window, n, b_lo, n_cand):
    """Candidate numbers (block - b_lo) of the history blocks in one head's
    token list, after checking that the list is sinks, whole 16-token
    blocks of candidates and the window, ascending and unique."""
    idx_g = np.asarray(idx_g, np.int64)
    assert np.all(np.diff(idx_g) > 0), "list not ascending and unique"
    assert np.array_equal(idx_g[:sinks], np.arange(sinks)), "sinks missing"
    if window:
        assert np.array_equal(idx_g[len(idx_g) - window:], np.arange(n - window, n)), "window missing"
    hist = idx_g[sinks:len(idx_g) - window]
    assert hist.size % 16 == 0
    blocks = hist.reshape(-1, 16)
    assert np.all(blocks == blocks[:, :1] + np.arange(16)) and np.all(blocks[:, 0] % 16 == 0), "partial blocks"
    c = blocks[:, 0] // 16 - b_lo
    assert np.all((c >= 0) & (c < n_cand)), "a kept block is not a candidate"
    return c


def is_valid_topk(scores, bands, kept, k):
    """Whether `kept` (candidate numbers) is a top-k of `scores` up to swaps
    within the bands.  Returns (ok, margin): margin = min over kept of
    (s + band) minus max over dropped of (s - band); ok iff margin >= 0."""
    kept = np.asarray(kept, np.int64)
    if kept.size != k or np.unique(kept).size != k:
        return False, -np.inf
    mask = np.zeros(scores.size, bool)
    mask[kept] = True
    if mask.all() or not mask.any():
        return True, np.inf
    margin = float((scores[mask] + bands[mask]).min() - (scores[~mask] - bands[~mask]).max())
    return margin >= 0, margin
