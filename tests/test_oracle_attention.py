"""Pins of the oracle's attention, score update and prompt importance (CPU).

Sources: DiffKV notes, "Background" (attention = softmax(q k^T / sqrt d)
weighting v; GQA shares a KV head among q heads), "Key observations" (the
same output written as coefficient softmax*|v| times unit vector v/|v|),
"KV compression policy" (importance = mean received attention, max over the
q heads of a KV head).
"""
import numpy as np
import pytest


def _np_attention(q, k, v):
    x = (k @ q) / np.sqrt(q.size)
    p = np.exp(x - x.max())
    p /= p.sum()
    return p @ v, p


def test_dense_matches_brute_force(orc):
    rng = np.random.default_rng(0)
    for n in (1, 2, 7, 50):
        q, k, v = rng.standard_normal(16), rng.standard_normal((n, 16)), rng.standard_normal((n, 16))
        ref, _ = _np_attention(q, k, v)
        assert np.allclose(orc.attention_dense(q, k, v), ref, rtol=1e-12, atol=1e-13)


def test_coefficient_unit_vector_identity(orc):
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal(32), rng.standard_normal((40, 32)), rng.standard_normal((40, 32)) * 3
    v[5] = 0.0  # a zero value vector contributes nothing either way
    a = orc.attention_dense(q, k, v)
    b = orc.attention_unit_vectors(q, k, v)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def _grid_token(rng, d, kbits, vbits):
    """K and V vectors lying exactly on their quantization grid (codes 0 and
    2^b-1 present, fp16-exact step and zero) so quantization is lossless."""
    def one(bits, step, zero):
        qmax = (1 << bits) - 1
        c = rng.integers(0, qmax + 1, d)
        c[rng.choice(d, 2, replace=False)] = [0, qmax]
        return (zero + step * c).astype(np.float32)
    return one(kbits, 2.0 ** -4, -8.0), one(vbits, 0.5, -3.0)


def _single_unit_state(orc, d, G, tiers_row, xk, xv, window=0, codec=None):
    N = tiers_row.size
    cfg = dict(head_dim=d, num_kv_heads=1, gqa_group=G, max_seq_len=N + 8, window=window,
               alpha_h=1.0, alpha_l=0.2)
    if codec is not None:
        cfg.update(hi_k_bits=codec[0], hi_v_bits=codec[1], lo_k_bits=codec[2], lo_v_bits=codec[3])
    st = orc.State(cfg, batch=1, num_pages=2 * N // 16 + 8)
    k = xk.astype(np.float16).view(np.uint16)[:, None, :]
    v = xv.astype(np.float16).view(np.uint16)[:, None, :]
    st.compact_prompt([0, N], k, v, np.zeros((1, N), np.float32), tiers_row[None, :])
    assert st.status[0] == 0
    return cfg, st


@pytest.mark.parametrize("d,codec", [(64, None), (128, None), (64, (4, 8, 2, 4)), (128, (8, 2, 4, 1))])
def test_lossless_cache_equals_textbook_attention(orc, d, codec):
    # codec: the tier widths (K high, V high, K low, V low); None: K8V4 / K4V2
    rng = np.random.default_rng(d + (sum(codec) if codec else 0))
    N, G = 90, 3
    tiers = rng.choice([orc.PRUNE, orc.LO, orc.HI], N).astype(np.uint8)
    xk = np.zeros((N, d), np.float32)
    xv = np.zeros((N, d), np.float32)
    w = codec or (8, 4, 4, 2)
    for t in range(N):
        kb, vb = (w[0], w[1]) if tiers[t] == orc.HI else (w[2], w[3])
        xk[t], xv[t] = _grid_token(rng, d, kb, vb)
    cfg, st = _single_unit_state(orc, d, G, tiers, xk, xv, codec=codec)
    q = rng.standard_normal((1, G, d)).astype(np.float16)
    out = st.decode_attn(q.view(np.uint16), [N])
    keep = tiers != orc.PRUNE
    for g in range(G):
        ref, _ = _np_attention(q[0, g].astype(np.float64), xk[keep].astype(np.float64),
                               xv[keep].astype(np.float64))
        assert np.allclose(out[0, g], ref, rtol=1e-6, atol=1e-6)


def test_one_token_and_equal_keys(orc):
    rng = np.random.default_rng(5)
    d = 64
    xk, xv = _grid_token(rng, d, 8, 4)
    cfg, st = _single_unit_state(orc, d, 2, np.array([orc.HI], np.uint8), xk[None], xv[None])
    q = rng.standard_normal((1, 2, d)).astype(np.float16).view(np.uint16)
    out = st.decode_attn(q, [1])
    assert np.array_equal(out[0, 0], xv) and np.array_equal(out[0, 1], xv)
    # equal keys: uniform weights, output is the mean of the values
    N = 20
    xks = np.repeat(xk[None], N, 0)
    xvs = np.stack([_grid_token(rng, d, 8, 4)[1] for _ in range(N)])
    cfg, st = _single_unit_state(orc, d, 1, np.full(N, orc.HI, np.uint8), xks, xvs)
    out = st.decode_attn(q[:, :1], [N])
    assert np.allclose(out[0, 0], xvs.astype(np.float64).mean(0), rtol=1e-6, atol=1e-6)


def test_slot_order_does_not_matter(orc):
    rng = np.random.default_rng(6)
    d, N = 64, 70
    xk = (rng.standard_normal((N, d)) * 2).astype(np.float16).astype(np.float32)
    xv = rng.standard_normal((N, d)).astype(np.float16).astype(np.float32)
    tiers = rng.choice([orc.LO, orc.HI], N).astype(np.uint8)
    perm = rng.permutation(N)
    q = rng.standard_normal((1, 2, d)).astype(np.float16).view(np.uint16)
    _, a = _single_unit_state(orc, d, 2, tiers, xk, xv)
    _, b = _single_unit_state(orc, d, 2, tiers[perm], xk[perm], xv[perm])
    oa, ob = a.decode_attn(q, [N]), b.decode_attn(q, [N])
    assert np.allclose(oa, ob, rtol=1e-6, atol=1e-7)


def test_score_update_mass_bounds(orc):
    # Per q head the softmax weights of all tokens but the query's own sum to
    # 1 - p_self, so the added mass (max over the group) lies in
    # [max_g (1 - p_self,g), G]; the own token's sum is unchanged.
    rng = np.random.default_rng(8)
    d, N, G = 64, 60, 4
    xk = rng.standard_normal((N, d)).astype(np.float16).astype(np.float32)
    xv = rng.standard_normal((N, d)).astype(np.float16).astype(np.float32)
    tiers = np.full(N, orc.HI, np.uint8)
    cfg, st = _single_unit_state(orc, d, G, tiers, xk, xv)
    before = {r["pos"]: r["score"] for _, _, r in st.unit_tokens(0, 0)}
    q = rng.standard_normal((1, G, d)).astype(np.float16)
    own = N - 1                              # query position = seq_len
    st.decode_attn(q.view(np.uint16), [own], update_scores=True)
    after = {r["pos"]: r["score"] for _, _, r in st.unit_tokens(0, 0)}
    delta = np.array([after[p] - before[p] for p in range(N)], np.float64)
    assert delta[own] == 0.0
    assert np.all(delta >= 0) and np.all(delta <= 1 + 1e-6)
    # dequantized keys as the cache holds them
    kh = np.stack([[orc.dequant(*r["kmeta"], int(c)) for c in r["k"]] for _, _, r in st.unit_tokens(0, 0)])
    pself = []
    for g in range(G):
        _, p = _np_attention(q[0, g].astype(np.float64), kh.astype(np.float64), np.zeros((N, 1)))
        pself.append(p[own])
    lo = max(1 - ps for ps in pself)
    assert lo - 1e-5 <= delta.sum() <= G + 1e-5


def test_score_update_worked_case(orc):
    # three tokens with equal keys, one q head: weights 1/3 each; the two
    # tokens before the query's own gain exactly fp32(1/3)
    d = 64
    rng = np.random.default_rng(9)
    xk, xv = _grid_token(rng, d, 8, 4)
    cfg, st = _single_unit_state(orc, d, 1, np.full(3, orc.HI, np.uint8),
                                 np.repeat(xk[None], 3, 0), np.repeat(xv[None], 3, 0))
    q = rng.standard_normal((1, 1, d)).astype(np.float16).view(np.uint16)
    st.decode_attn(q, [2], update_scores=True)
    sc = sorted((r["pos"], r["score"]) for _, _, r in st.unit_tokens(0, 0))
    assert sc == [(0, np.float32(1 / 3)), (1, np.float32(1 / 3)), (2, 0.0)]


def test_importance_from_queries(orc):
    rng = np.random.default_rng(10)
    d, H, G, N = 64, 2, 3, 30
    cfg = dict(head_dim=d, num_kv_heads=H, gqa_group=G, max_seq_len=64, window=0, alpha_h=1.0, alpha_l=0.2)
    k = rng.standard_normal((N, H, d)).astype(np.float16)
    qp = rng.standard_normal((1, 5, H * G, d)).astype(np.float16)
    sc = orc.importance_from_queries(cfg, [0, N], k.view(np.uint16), qp.view(np.uint16))
    for h in range(H):
        ref = np.zeros(N)
        for qi in range(5):
            ps = [_np_attention(qp[0, qi, h * G + g].astype(np.float64), k[:, h].astype(np.float64),
                                np.zeros((N, 1)))[1] for g in range(G)]
            ref += np.max(ps, axis=0)
        assert np.allclose(sc[h], ref / 5, rtol=1e-6)
    # equal keys -> every token receives 1/N
    keq = np.repeat(k[:1], N, 0)
    sc = orc.importance_from_queries(cfg, [0, N], keq.view(np.uint16), qp.view(np.uint16))
    assert np.allclose(sc, 1 / N, rtol=1e-6)
    # one q head per group, one probe: the scores are one softmax, summing to 1
    cfg1 = dict(cfg, gqa_group=1)
    sc = orc.importance_from_queries(cfg1, [0, N], k.view(np.uint16), qp[:, :1, :H].view(np.uint16))
    assert np.allclose(sc.sum(1), 1.0, rtol=1e-6)


def _gqa_worked_case(orc, d, seq_len_own):
    """Five high tokens, constant keys (lossless: zero scale, zero = the
    value): token 2 holds +1 in every dim, the others -1.  Two q heads of one
    group: head 0 = 3 in every dim, so its logits are +-3 sqrt(d) and token 2
    takes all its weight (the other weights are below e^-48, far under fp64
    resolution next to 1); head 1 = 0, so its weights are exactly 1/5.  The
    group's weight of a token is the max over the heads (DiffKV notes, "KV
    compression policy": GQA scores combined with max): token 2 gains 1.0,
    every other token exactly fp32(1/5).  A sum over the heads would give
    token 2 1.2, a mean 0.6 (and the others 0.1); head 0 alone would give the
    others 0, head 1 alone token 2 0.2."""
    n, G = 5, 2
    xk = np.where(np.arange(n)[:, None] == 2, 1.0, -1.0) * np.ones((n, d))
    rng = np.random.default_rng(12)
    xv = np.stack([_grid_token(rng, d, 8, 4)[1] for _ in range(n)])
    cfg, st = _single_unit_state(orc, d, G, np.full(n, orc.HI, np.uint8), xk.astype(np.float32), xv)
    q = np.zeros((1, G, d), np.float16)
    q[0, 0] = 3.0
    before = {r["pos"]: r["score"] for _, _, r in st.unit_tokens(0, 0)}
    st.decode_attn(q.view(np.uint16), [seq_len_own], update_scores=True)
    after = {r["pos"]: r["score"] for _, _, r in st.unit_tokens(0, 0)}
    return n, before, after, q


@pytest.mark.parametrize("d", [64, 128])
def test_score_update_max_over_group_worked_case(orc, d):
    n, before, after, _ = _gqa_worked_case(orc, d, seq_len_own=4)
    assert all(before[p] == 0.0 for p in range(n))
    # token 4 is the query's own (position seq_len): unchanged
    expect = {0: np.float32(0.2), 1: np.float32(0.2), 2: np.float32(1.0), 3: np.float32(0.2), 4: np.float32(0.0)}
    assert {p: np.float32(after[p]) for p in range(n)} == expect


def test_score_update_equals_numpy_max_elementwise(orc):
    # Random keys, G = 4: each token's increment equals max over the group of
    # the numpy softmax weights (dequantized keys, fp64), elementwise; the
    # sum over the group is far from it.
    rng = np.random.default_rng(8)
    d, N, G = 64, 60, 4
    xk = rng.standard_normal((N, d)).astype(np.float16).astype(np.float32)
    xv = rng.standard_normal((N, d)).astype(np.float16).astype(np.float32)
    cfg, st = _single_unit_state(orc, d, G, np.full(N, orc.HI, np.uint8), xk, xv)
    before = {r["pos"]: r["score"] for _, _, r in st.unit_tokens(0, 0)}
    q = rng.standard_normal((1, G, d)).astype(np.float16)
    own = N - 1
    st.decode_attn(q.view(np.uint16), [own], update_scores=True)
    after = {r["pos"]: r["score"] for _, _, r in st.unit_tokens(0, 0)}
    delta = np.array([after[p] - before[p] for p in range(N)], np.float64)
    kh = np.stack([[orc.dequant(*r["kmeta"], int(c)) for c in r["k"]]
                   for _, _, r in sorted(st.unit_tokens(0, 0), key=lambda e: e[2]["pos"])])
    ps = np.stack([_np_attention(q[0, g].astype(np.float64), kh.astype(np.float64), np.zeros((N, 1)))[1]
                   for g in range(G)])
    assert np.allclose(delta[:own], ps.max(0)[:own], rtol=1e-6, atol=1e-7)
    assert np.abs(delta[:own] - ps.sum(0)[:own]).max() > 1e-2
