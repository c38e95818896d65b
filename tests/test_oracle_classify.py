"""Pins of the oracle's token classification (CPU only).

Source: DiffKV notes, "Approach" and "KV compression policy": high if the
mean score exceeds alpha_h/N, low if it lies in [alpha_l/N, alpha_h/N],
pruned below alpha_l/N; the last W tokens are always high.  Variants from
the same section: the prompt-phase paragraph's alpha/i (i-th token), and the
extensibility paragraph's per-head thresholds.
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


# --- the sequence-length-adaptive rule: the i-th prompt token against alpha/i
# ("KV compression policy", prompt-phase paragraph; i counts from 1)

def test_alpha_i_rule_dyadic(orc):
    # N = 8, W = 0, alpha_h = 1, alpha_l = 1/2.  Thresholds per position p
    # (i = p + 1): high > 1/i, low >= 1/(2i).
    #   p=0 (i=1): 0.75 in [1/2, 1]             -> low    (alpha/N: high)
    #   p=1 (i=2): 0.5 == 1/2, not above         -> low    (alpha/N: high)
    #   p=2 (i=3): 0.125 < 1/6                   -> pruned (alpha/N: low)
    #   p=3 (i=4): 0.25 + ulp > 1/4              -> high
    #   p=4 (i=5): fp32(0.1) lies just above 1/10 = alpha_l/i -> low
    #   p=5 (i=6): 0.0625 < 1/12                 -> pruned (alpha/N: low)
    #   p=6 (i=7): 0.2 > 1/7                     -> high
    #   p=7 (i=8): 0.0625 == 1/16 = alpha_l/i    -> low
    up = float(np.nextafter(np.float32(0.25), np.float32(1)))
    s = np.array([[0.75, 0.5, 0.125, up, 0.1, 0.0625, 0.2, 0.0625]], np.float32)
    c = _cfg(alpha_h=1.0, alpha_l=0.5, prompt_rule=orc.RULE_ALPHA_I)
    tiers, counts = orc.classify(c, np.array([0, 8]), s)
    assert tiers.tolist() == [[orc.LO, orc.LO, orc.PRUNE, orc.HI, orc.LO, orc.PRUNE, orc.HI, orc.LO]]
    assert counts.tolist() == [[[2, 4]]]
    # the length rule on the same scores: high > 1/8, low >= 1/16
    tiers_n, _ = orc.classify(_cfg(alpha_h=1.0, alpha_l=0.5), np.array([0, 8]), s)
    assert tiers_n.tolist() == [[orc.HI, orc.HI, orc.LO, orc.HI, orc.LO, orc.LO, orc.HI, orc.LO]]


def test_alpha_i_rule_window_and_low_tier_off(orc):
    # the window still forces the newest W tokens high; with the low tier off a
    # token is high iff s i >= alpha_l
    s = np.array([[0.0, 0.3, 0.3, 0.0, 0.0]], np.float32)
    c = _cfg(window=2, alpha_l=0.5, lo_enabled=0, alpha_h=0.0, prompt_rule=orc.RULE_ALPHA_I)
    tiers, counts = orc.classify(c, np.array([0, 5]), s)
    # p=1 (i=2): 0.6 >= 0.5 high; p=2 (i=3): 0.9 high; p=0: 0 pruned; p=3,4 window
    assert tiers.tolist() == [[orc.PRUNE, orc.HI, orc.HI, orc.HI, orc.HI]]
    assert counts.tolist() == [[[4, 0]]]


@pytest.mark.parametrize("lo_enabled", [1, 0])
def test_alpha_i_is_alpha_n_of_the_prefix(orc, lo_enabled):
    # With W = 0 the i-th token's alpha/i decision is the alpha/N decision of
    # the last token of the length-i prefix; and since i <= N, alpha/i is never
    # laxer than alpha/N (tier under alpha/i <= tier under alpha/N).
    rng = np.random.default_rng(3)
    H, lens = 2, [37, 1, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    total = int(cu[-1])
    s = (rng.random((H, total)) ** 3 / 8).astype(np.float32)
    c = _cfg(num_kv_heads=H, alpha_h=1.0, alpha_l=0.2, lo_enabled=lo_enabled)
    t_i, counts_i = orc.classify(dict(c, prompt_rule=orc.RULE_ALPHA_I), cu, s)
    t_n, _ = orc.classify(c, cu, s)
    assert np.all(t_i <= t_n)
    for r, N in enumerate(lens):
        for p in range(N):
            ci = np.array([0, p + 1])
            pref = np.ascontiguousarray(s[:, cu[r]:cu[r] + p + 1])
            t_p, _ = orc.classify(c, ci, pref)
            assert np.array_equal(t_p[:, p], t_i[:, cu[r] + p]), (r, p)
    for r in range(len(lens)):
        for h in range(H):
            seg = t_i[h, cu[r]:cu[r + 1]]
            assert counts_i[r, h].tolist() == [np.sum(seg == orc.HI), np.sum(seg == orc.LO)]


# --- per-head thresholds ("KV compression policy", extensibility paragraph:
# one shared pair by default, each head's own pair as an option)

def test_per_head_thresholds_dyadic(orc):
    # H = 2, N = 4, W = 0: head 0 uses (1, 1/4) -> high > 1/4, low >= 1/16;
    # head 1 uses (2, 1) -> high > 1/2, low >= 1/4.  The shared pair is unused.
    s = np.array([[0.3, 0.25, 0.0625, 0.05],
                  [0.6, 0.5, 0.25, 0.2]], np.float32)
    c = _cfg(num_kv_heads=2, alpha_h=100.0, alpha_l=50.0,
             alpha_h_head=[1.0, 2.0], alpha_l_head=[0.25, 1.0])
    tiers, counts = orc.classify(c, np.array([0, 4]), s)
    assert tiers.tolist() == [[orc.HI, orc.LO, orc.LO, orc.PRUNE],
                              [orc.HI, orc.LO, orc.LO, orc.PRUNE]]
    assert counts.tolist() == [[[1, 2], [1, 2]]]


@pytest.mark.parametrize("rule", [0, 1])
def test_per_head_equals_shared_run_per_head(orc, rule):
    # each head's decisions with per-head arrays are those of a shared-pair
    # run whose pair is that head's
    rng = np.random.default_rng(5)
    H, lens = 3, [50, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    s = (rng.random((H, int(cu[-1]))) ** 3 / 8).astype(np.float32)
    ah, al = [0.5, 1.0, 3.0], [0.0, 0.2, 0.7]
    c = _cfg(num_kv_heads=H, window=4, prompt_rule=rule, alpha_h_head=ah, alpha_l_head=al)
    t, counts = orc.classify(c, cu, s)
    for h in range(H):
        th, ch = orc.classify(_cfg(num_kv_heads=H, window=4, prompt_rule=rule,
                                   alpha_h=ah[h], alpha_l=al[h]), cu, s)
        assert np.array_equal(t[h], th[h]) and np.array_equal(counts[:, h], ch[:, h])
    assert len({tuple(t[h]) for h in range(H)}) == H       # the heads do differ


def test_policy_config_rejections(orc):
    cu, s = np.array([0, 2]), np.zeros((2, 2), np.float32)
    base = _cfg(num_kv_heads=2)
    for bad in (dict(prompt_rule=2), dict(prompt_rule=-1),
                dict(alpha_h_head=[1.0, 1.0]),                          # one array only
                dict(alpha_h_head=[1.0, 0.1], alpha_l_head=[0.5, 0.2]),  # alpha_l > alpha_h
                dict(alpha_h_head=[1.0, 1.0], alpha_l_head=[-0.5, 0.2])):
        with pytest.raises(ValueError):
            orc.classify(dict(base, **bad), cu, s)
    # alpha_l > alpha_h is fine with the low tier closed
    orc.classify(dict(base, lo_enabled=0, alpha_h_head=[1.0, 0.1], alpha_l_head=[0.5, 0.2]), cu, s)
