"""Pins of the oracle's per-page key bounds and page scores (FlexiCache page,
"3.2 KV页评分机制", after Quest: per page the per-dimension min and max key;
a query's page score is the largest dot product it could have with any key
of the page, sum_i max(q_i kmin_i, q_i kmax_i); the group's q heads combined
with max).  Keys are the dequantized keys the cache holds."""
import numpy as np
import pytest


def _state(orc, rng, d, G, N, tiers):
    cfg = dict(head_dim=d, num_kv_heads=1, gqa_group=G, max_seq_len=N + 8, window=0, alpha_h=1.0, alpha_l=0.2)
    st = orc.State(cfg, batch=1, num_pages=2 * N // 16 + 8)
    k = (rng.standard_normal((N, 1, d)) * 2).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((N, 1, d)).astype(np.float16).view(np.uint16)
    st.compact_prompt([0, N], k, v, np.zeros((1, N), np.float32), tiers[None, :])
    assert st.status[0] == 0
    return cfg, st


def _page_keys(orc, st):
    """{page id: [dequantized keys of its retained slots]} for unit (0, 0)."""
    L = st.page_table.shape[-1]
    out = {}
    for tier, slot, rec in st.unit_tokens(0, 0):
        pid = int(st.page_table[0, 0, slot // 16] if tier == orc.HI else st.page_table[0, 0, L - 1 - slot // 32])
        out.setdefault(pid, []).append([orc.dequant(*rec["kmeta"], int(c)) for c in rec["k"]])
    return {p: np.array(v, np.float32) for p, v in out.items()}


@pytest.mark.parametrize("d", [64, 128])
def test_bounds_equal_brute_force_min_max(orc, d):
    rng = np.random.default_rng(d)
    N = 150
    tiers = rng.choice([orc.PRUNE, orc.LO, orc.HI], N).astype(np.uint8)
    cfg, st = _state(orc, rng, d, 2, N, tiers)
    b = st.page_bounds()
    for pid, keys in _page_keys(orc, st).items():
        assert np.array_equal(b[pid, 0], keys.min(0)) and np.array_equal(b[pid, 1], keys.max(0))


def test_score_bounds_every_key_and_single_token_is_exact(orc):
    rng = np.random.default_rng(3)
    d, G, N = 64, 3, 120
    tiers = rng.choice([orc.LO, orc.HI], N).astype(np.uint8)
    cfg, st = _state(orc, rng, d, G, N, tiers)
    q = rng.standard_normal((1, G, d)).astype(np.float16)
    b = st.page_bounds()
    sc = st.page_scores(q.view(np.uint16), [N], b)[0, 0]
    L = st.page_table.shape[-1]
    for pid, keys in _page_keys(orc, st).items():
        t = int(np.flatnonzero(st.page_table[0, 0] == pid)[0])
        best = float((keys.astype(np.float64) @ q[0].astype(np.float64).T).max())   # every key, every head
        assert sc[t] >= best - 1e-6 * abs(best)       # an upper bound of every q.k in the page
    empty = [t for t in range(L) if not (t < st.tier_state[0, 0, 2] or t >= L - st.tier_state[0, 0, 3])]
    assert np.all(np.isneginf(sc[empty]))
    # a page with one token: the bound is that token's dot product (max over the group)
    cfg1, st1 = _state(orc, rng, d, G, 1, np.array([orc.HI], np.uint8))
    k1 = _page_keys(orc, st1)
    (pid, keys), = k1.items()
    s1 = st1.page_scores(q.view(np.uint16), [1], st1.page_bounds())[0, 0, 0]
    assert s1 == np.float32((keys.astype(np.float64) @ q[0].astype(np.float64).T).max())


def test_opposite_corners_closed_form(orc):
    # two keys +a and -a in one page: min/max are -|a|, |a| per dimension, so
    # the bound is sum_i |q_i a_i| (the group's max)
    d, G = 64, 2
    rng = np.random.default_rng(4)
    a = np.round(rng.uniform(-3, 3, d) * 8) / 8                 # fp16-exact
    cfg = dict(head_dim=d, num_kv_heads=1, gqa_group=G, max_seq_len=16, window=0, alpha_h=1.0, alpha_l=0.2)
    st = orc.State(cfg, batch=1, num_pages=4)
    k = np.stack([a, -a]).astype(np.float16).view(np.uint16)[:, None, :]
    st.compact_prompt([0, 2], k, k, np.zeros((1, 2), np.float32), np.full((1, 2), orc.HI, np.uint8))
    keys = _page_keys(orc, st)[int(st.page_table[0, 0, 0])].astype(np.float64)
    q = rng.standard_normal((1, G, d)).astype(np.float16)
    s = st.page_scores(q.view(np.uint16), [2], st.page_bounds())[0, 0, 0]
    lo, hi = keys.min(0), keys.max(0)
    ref = max(float(np.sum(np.maximum(q[0, g] * lo, q[0, g] * hi))) for g in range(G))
    assert s == np.float32(ref)
    # and with the dequantized keys symmetric up to the codec, |q| . |a| within its error
    ref_abs = max(float(np.sum(np.abs(q[0, g].astype(np.float64) * a))) for g in range(G))
    assert abs(s - ref_abs) <= 0.05 * ref_abs


def _levels_state(orc, rng, K, d=64, G=2, N=300):
    """A one-unit cache of K precision levels from the oracle's prompt
    compaction (codes spread over every level and pruned)."""
    base = dict(head_dim=d, num_kv_heads=1, gqa_group=G, max_seq_len=N + 8, window=0, alpha_h=1.0, alpha_l=0.2,
                hi_k_bits=8, hi_v_bits=8, lo_k_bits=4, lo_v_bits=2, num_levels=K)
    if K == 3:
        base.update(alpha_mid=[0.5], mid_k_bits=[8], mid_v_bits=[4])
    else:
        base.update(alpha_mid=[0.6, 0.4], mid_k_bits=[8, 2], mid_v_bits=[4, 2])
    st = orc.State(base, batch=1, num_pages=2 * N // 16 + 8)
    k = (rng.standard_normal((N, 1, d)) * 2).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((N, 1, d)).astype(np.float16).view(np.uint16)
    codes = rng.integers(0, K + 1, N).astype(np.uint8)            # K - level, 0 pruned
    st.compact_prompt([0, N], k, v, np.zeros((1, N), np.float32), codes[None, :])
    assert st.status[0] == 0
    return base, st


def _level_page_keys(orc, st):
    """{page id: [dequantized keys of its retained slots]} for unit (0, 0) of
    a K-level cache."""
    out = {}
    for lv, slot, rec in st.unit_tokens(0, 0):
        T = 16 if lv == 0 else 32
        pid = st.level_page(0, 0, lv, slot // T)
        out.setdefault(pid, []).append([orc.dequant(*rec["kmeta"], int(c)) for c in rec["k"]])
    return {p: np.array(v, np.float32) for p, v in out.items()}


@pytest.mark.parametrize("K", [3, 4])
def test_levels_bounds_brute_force_and_score_bound(orc, K):
    """K precision levels: every live page of every level (its own codec and
    page size) gets the per-dimension min / max of its dequantized keys; the
    page score bounds every q.k in the page, empty entries are -inf."""
    rng = np.random.default_rng(40 + K)
    cfg, st = _levels_state(orc, rng, K)
    b = st.page_bounds()
    keys = _level_page_keys(orc, st)
    assert len(keys) >= K  # pages of several levels
    for pid, kk in keys.items():
        assert np.array_equal(b[pid, 0], kk.min(0)) and np.array_equal(b[pid, 1], kk.max(0))
    q = rng.standard_normal((1, cfg["gqa_group"], cfg["head_dim"])).astype(np.float16)
    sc = st.page_scores(q.view(np.uint16), [300], b)[0, 0]
    live = set()
    for pid, kk in keys.items():
        t = int(np.flatnonzero(st.page_table[0, 0] == pid)[0])
        live.add(t)
        best = float((kk.astype(np.float64) @ q[0].astype(np.float64).T).max())
        assert sc[t] >= best - 1e-6 * abs(best)
    dead = [t for t in range(sc.size) if t not in live]
    assert np.all(np.isneginf(sc[dead]))
    assert np.all(np.isneginf(st.page_scores(q.view(np.uint16), [0], b)))  # inactive request


def test_levels_single_token_page_score_is_exact(orc):
    """A page of one token at a middle level: its score is that token's dot
    product (the group's max)."""
    rng = np.random.default_rng(7)
    cfg = dict(head_dim=64, num_kv_heads=1, gqa_group=3, max_seq_len=24, window=0, alpha_h=1.0, alpha_l=0.2,
               hi_k_bits=8, hi_v_bits=8, lo_k_bits=4, lo_v_bits=2, num_levels=3, alpha_mid=[0.5],
               mid_k_bits=[8], mid_v_bits=[4])
    st = orc.State(cfg, batch=1, num_pages=8)
    k = (rng.standard_normal((1, 1, 64)) * 2).astype(np.float16).view(np.uint16)
    st.compact_prompt([0, 1], k, k, np.zeros((1, 1), np.float32), np.array([[2]], np.uint8))  # level 1
    (pid, kk), = _level_page_keys(orc, st).items()
    q = rng.standard_normal((1, 3, 64)).astype(np.float16)
    s = st.page_scores(q.view(np.uint16), [1], st.page_bounds())[0, 0]
    t = int(np.flatnonzero(st.page_table[0, 0] == pid)[0])
    assert s[t] == np.float32((kk.astype(np.float64) @ q[0].astype(np.float64).T).max())
