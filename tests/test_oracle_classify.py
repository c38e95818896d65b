"""Pins of the oracle's token classification (CPU only).

Source: DiffKV notes, "Approach" and "KV compression policy": high if the
mean score exceeds alpha_h/N, low if it lies in [alpha_l/N, alpha_h/N],
pruned below alpha_l/N; the last W tokens are always high.
"""
import math

import numpy as np
import pytest


def _cfg(**kw):
    c = dict(head_dim=64, num_kv_heads=1, gqa_group=1, max_seq_len=1 << 20, window=0,
             alpha_h=1.0, alpha_l=0.25, lo_enabled=1)
    c.update(kw)
    return c


def test_threshold_edges_dyadic(orc):
    # N = 4, alpha_h = 1 -> 1/4 ; alpha_l = 1/4 -> 1/16 (exact in fp32)
    up = np.nextafter(np.float32(0.25), np.float32(1))
    dn = np.nextafter(np.float32(1 / 16), np.float32(0))
    s = np.array([[0.25, up, 1 / 16, dn]], np.float32)
    tiers, counts = orc.classify(_cfg(), np.array([0, 4]), s)
    assert tiers.tolist() == [[orc.LO, orc.HI, orc.LO, orc.PRUNE]]
    assert counts.tolist() == [[[1, 2]]]


def test_window_override(orc):
    s = np.zeros((1, 6), np.float32)
    tiers, counts = orc.classify(_cfg(window=2), np.array([0, 6]), s)
    assert tiers.tolist() == [[0, 0, 0, 0, 2, 2]]
    # window longer than the prompt: everything high
    tiers, _ = orc.classify(_cfg(window=64), np.array([0, 6]), s)
    assert np.all(tiers == orc.HI)


def test_low_tier_disabled(orc):
    # alpha_l/N = 1/16: at or above -> high, below -> pruned; alpha_h unused
    dn = np.nextafter(np.float32(1 / 16), np.float32(0))
    s = np.array([[1 / 16, dn, 0.2, 0.9]], np.float32)
    tiers, counts = orc.classify(_cfg(lo_enabled=0, alpha_h=0.0), np.array([0, 4]), s)
    assert tiers.tolist() == [[orc.HI, orc.PRUNE, orc.HI, orc.HI]]
    assert counts.tolist() == [[[3, 0]]]


def test_ragged_batch_layout(orc):
    # head-major [H, sum N]; each request uses its own N in alpha/N
    c = _cfg(num_kv_heads=2)
    cu = np.array([0, 2, 6])
    s = np.array([[0.6, 0.3, 0.2, 0.2, 0.0, 0.3],
                  [0.4, 0.6, 0.1, 0.05, 0.25, 0.3]], np.float32)
    tiers, counts = orc.classify(c, cu, s)
    # request 0 (N=2): hi > 0.5, lo >= 0.125 ; request 1 (N=4): hi > 0.25, lo >= 0.0625
    assert tiers.tolist() == [[2, 1, 1, 1, 0, 2], [1, 2, 1, 0, 1, 2]]
    assert counts.tolist() == [[[1, 1], [1, 1]], [[1, 2], [1, 2]]]


@pytest.mark.parametrize("s_exp,N", [(1.1, 4096), (0.8, 1000), (1.6, 32768)])
def test_zipf_counts_closed_form(orc, s_exp, N):
    # Zipf mass p_k = k^-s / H_N(s): since p_k decreases with the rank, the
    # number of tokens above alpha/N is the number of ranks k with
    # k < (N / (alpha H_N))^(1/s).
    Hn = math.fsum(k ** -s_exp for k in range(1, N + 1))
    p = np.array([k ** -s_exp / Hn for k in range(1, N + 1)]).astype(np.float32)
    rng = np.random.default_rng(0)
    perm = rng.permutation(N)
    c = _cfg(alpha_h=1.0, alpha_l=0.2)
    tiers, counts = orc.classify(c, np.array([0, N]), p[perm][None, :])
    for alpha, expect_idx in ((1.0, 0), (0.2, None)):
        x = (N / (alpha * Hn)) ** (1 / s_exp)
        n_above = math.ceil(x) - 1 if x == int(x) else math.floor(x)
        n_above = min(n_above, N)
        if expect_idx == 0:
            assert counts[0, 0, 0] == n_above
        else:
            assert counts[0, 0, 0] + counts[0, 0, 1] == n_above
    assert counts[0, 0, 0] == int(np.sum(tiers == orc.HI))
