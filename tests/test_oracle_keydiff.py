"""Pins of the oracle's query-free importance (KeyDiff page, "方法细节":
the anchor is the mean of the unit's normalized keys -- or of the raw keys,
the page's simplification -- and a key's eviction score is its cosine to
the anchor, the least similar kept).  Reading taken to feed classification:
w_i = 1 - cos(anchor, k_i), normalized over the unit (uniform when every key
is parallel to the anchor)."""
import numpy as np
import pytest


def _cfg(d, H):
    return dict(head_dim=d, num_kv_heads=H, gqa_group=1, max_seq_len=4096, window=0, alpha_h=1.0, alpha_l=0.2)


def test_two_directions_closed_form(orc):
    # n_a keys along e_a (norm 2) and n_b along e_b (norm 3): the normalized
    # anchor is (n_a e_a + n_b e_b) / n, so cos = n_a / sqrt(n_a^2 + n_b^2)
    # for the first group and n_b / ... for the second
    d, na, nb = 64, 5, 12
    k = np.zeros((na + nb, 1, d), np.float16)
    k[:na, 0, 3] = 2.0
    k[na:, 0, 40] = 3.0
    sc = orc.keydiff_scores(_cfg(d, 1), [0, na + nb], k.view(np.uint16))[0]
    r = np.hypot(na, nb)
    wa, wb = 1 - na / r, 1 - nb / r
    tot = na * wa + nb * wb
    assert np.allclose(sc[:na], wa / tot, rtol=1e-6) and np.allclose(sc[na:], wb / tot, rtol=1e-6)
    # the raw-key anchor weighs the norms: (2 n_a e_a + 3 n_b e_b) / n
    sc = orc.keydiff_scores(_cfg(d, 1), [0, na + nb], k.view(np.uint16), anchor_raw=True)[0]
    r = np.hypot(2 * na, 3 * nb)
    wa, wb = 1 - 2 * na / r, 1 - 3 * nb / r
    tot = na * wa + nb * wb
    assert np.allclose(sc[:na], wa / tot, rtol=1e-6) and np.allclose(sc[na:], wb / tot, rtol=1e-6)


def test_parallel_keys_uniform_and_zero_key(orc):
    d, N = 64, 9
    rng = np.random.default_rng(1)
    v = rng.standard_normal(d)
    k = (np.outer(rng.uniform(0.5, 2.0, N), v)).astype(np.float16)[:, None, :]
    sc = orc.keydiff_scores(_cfg(d, 1), [0, N], k.view(np.uint16))[0]
    # every key parallel to the anchor up to fp16 rounding: w ~ 0 for all;
    # the scores stay a distribution
    assert abs(sc.sum() - 1.0) < 1e-6
    k = np.zeros((N, 1, d), np.float16)
    sc = orc.keydiff_scores(_cfg(d, 1), [0, N], k.view(np.uint16))[0]
    assert np.allclose(sc, 1.0 / N)                   # zero keys: cos 0, w = 1 each


def test_anchor_cosine_equals_pairwise_definition(orc):
    # The page's O(n^2) definition scores key i by -sum_j CosSim(k_i, k_j).
    # With the normalized anchor mu, sum_j CosSim(k_i, k_j) = n |mu| cos(mu, k_i)
    # and |mu|^2 = sum_ij CosSim_ij / n^2: the oracle's cosines follow from
    # the pairwise matrix alone.
    rng = np.random.default_rng(2)
    d, H = 64, 2
    lens = [30, 7, 51]
    cu = np.concatenate([[0], np.cumsum(lens)])
    k = (rng.standard_normal((cu[-1], H, d)) + 0.7).astype(np.float16)
    sc = orc.keydiff_scores(_cfg(d, H), cu, k.view(np.uint16))
    for r, n in enumerate(lens):
        for h in range(H):
            K = k[cu[r]:cu[r + 1], h].astype(np.float64)
            Kh = K / np.linalg.norm(K, axis=1, keepdims=True)
            C = Kh @ Kh.T
            mu_norm = np.sqrt(C.sum()) / n
            cos = C.sum(1) / (n * mu_norm)
            w = 1 - cos
            assert np.allclose(sc[h, cu[r]:cu[r + 1]], w / w.sum(), rtol=1e-6, atol=1e-9)
            # the ranking is the page's topk(-CosSim(K) 1) ranking
            assert np.array_equal(np.argsort(-sc[h, cu[r]:cu[r + 1]], kind="stable"),
                                  np.argsort(C.sum(1), kind="stable"))
