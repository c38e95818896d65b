"""Pins of the oracle's K-level extension (CPU only).

Source: DiffKV notes, "KV compression policy" (extensibility paragraph: the
policy allows more than two quantization levels) and "Memory management"
(generation workflow: extra levels are supported by combining unidirectional
or bidirectional page tables).  The pages name the extension without its
details; the readings taken are stated in the oracle (levels section) and
pinned here by:
  * the two-tier case: the K-level code with K = 2 must reproduce the
    two-tier oracle (itself pinned by the Fig 6 worked example, the set model
    and the codec tests) byte for byte over prompts, hundreds of steps,
    attention with score updates, release and re-admission;
  * a set model of the K-level step written from the readings (positions per
    level, exact rational means, no slots or pages), run for hundreds of
    steps with every policy case occurring;
  * worked examples of the classification boundaries and of the generalized
    Fig 6 block placement (frees and extra pages) and release order;
  * attention on a lossless grid (dequantized values equal the inputs)
    against numpy softmax attention over the retained tokens.
"""
from fractions import Fraction

import numpy as np
import pytest

from tests.invariants import check_pool_invariants


# thresholds close together, so that tokens cross several levels between two
# visits and every case of the step occurs within a few hundred steps
def _cfg3(**over):
    c = dict(head_dim=64, num_kv_heads=2, gqa_group=2, max_seq_len=700, window=6, alpha_h=1.0, alpha_l=0.75,
             num_levels=3, alpha_mid=[0.85], mid_k_bits=[8], mid_v_bits=[2],
             hi_k_bits=8, hi_v_bits=8, lo_k_bits=4, lo_v_bits=2)
    c.update(over)
    return c


def _cfg4(**over):
    c = _cfg3(num_levels=4, alpha_mid=[0.9, 0.8], alpha_l=0.7, mid_k_bits=[8, 4], mid_v_bits=[4, 4])
    c.update(over)
    return c


def _prompt_inputs(rng, H, d, lens, sharp=4):
    cu = np.concatenate([[0], np.cumsum(lens)])
    total = int(cu[-1])
    scale = np.ones(d, np.float32)
    scale[[3, 17]] = 8.0
    k = (rng.standard_normal((total, H, d)) * scale).astype(np.float16).view(np.uint16)
    v = (rng.standard_normal((total, H, d)) * scale).astype(np.float16).view(np.uint16)
    sc = (rng.random((H, total)) ** sharp).astype(np.float32)
    sc /= sc.sum(1, keepdims=True) / 4
    return cu, k, v, sc, scale


def _states_equal(a, b, what):
    assert np.array_equal(a.tier_state, b.tier_state), what
    assert np.array_equal(a.page_table, b.page_table), what
    assert np.array_equal(a.free_list, b.free_list), what
    assert np.array_equal(a.ptr, b.ptr) and np.array_equal(a.status, b.status), what
    assert np.array_equal(a.pages, b.pages), what


# two-tier case code -> K-level (t_c class, victim class); 14 pruned, 15 none
_BR_MAP = {1: (15, 15), 2: (0, 0), 3: (0, 1), 4: (0, 14), 5: (1, None), 6: (1, 14), 7: (14, 15)}


@pytest.mark.parametrize("lo_enabled,codec", [(1, None), (0, None), (1, (4, 8, 2, 4))])
def test_levels_with_two_tiers_equal_the_two_tier_oracle(orc, lo_enabled, codec):
    rng = np.random.default_rng(11 + lo_enabled)
    d, H, G, B, W = 64, 2, 2, 3, 6
    cfg = dict(head_dim=d, num_kv_heads=H, gqa_group=G, max_seq_len=900, window=W, alpha_h=1.0, alpha_l=0.3,
               lo_enabled=lo_enabled)
    if codec:
        cfg.update(hi_k_bits=codec[0], hi_v_bits=codec[1], lo_k_bits=codec[2], lo_v_bits=codec[3])
    lens = np.array([60, 3, 33])
    cu, k, v, sc, scale = _prompt_inputs(rng, H, d, lens)
    t2, c2 = orc.classify(cfg, cu, sc)
    tk, ck = orc.classify(cfg, cu, sc, levels_impl=True)
    assert np.array_equal(t2, tk) and np.array_equal(c2, ck)
    a, b = orc.State(cfg, B, 300), orc.State(cfg, B, 300)
    a.compact_prompt(cu, k, v, sc, t2)
    b.compact_prompt(cu, k, v, sc, t2, levels_impl=True)
    _states_equal(a, b, "prompt")
    seq = lens.astype(np.int32).copy()
    seen = set()
    for step in range(150):
        kn = (rng.standard_normal((B, H, d)) * scale).astype(np.float16).view(np.uint16)
        vn = (rng.standard_normal((B, H, d)) * scale).astype(np.float16).view(np.uint16)
        ba = a.compact_step(seq, kn, vn, branches=True)
        bb = b.compact_step(seq, kn, vn, branches=True, levels_impl=True)
        _states_equal(a, b, f"step {step}")
        for x, y in zip(ba.ravel(), bb.ravel()):
            tc, vc = _BR_MAP[int(x) & 15]
            assert (int(y) & 15) == tc and (vc is None or ((int(y) >> 4) & 15) == vc), (x, y)
            tier = (int(x) >> 4) & 3
            assert ((int(y) >> 8) & 15) == {0: 0, 2: 1, 1: 2}[tier], (x, y)
            seen.add(int(x) & 15)
        q = (rng.standard_normal((B, H * G, d)) * 3).astype(np.float16).view(np.uint16)
        oa = a.decode_attn(q, seq, update_scores=True)
        ob = b.decode_attn(q, seq, update_scores=True, levels_impl=True)
        assert np.array_equal(oa, ob)
        _states_equal(a, b, f"attention {step}")
        seq += 1
    assert {2, 7} <= seen and (not lo_enabled or {3, 5, 6} <= seen), seen
    mask = np.array([1, 0, 1], np.uint8)
    a.release(mask)
    b.release(mask, levels_impl=True)
    _states_equal(a, b, "release")
    lens2 = np.array([50, 0, 17])
    cu2, k2, v2, sc2, _ = _prompt_inputs(rng, H, d, lens2)
    t2b, _ = orc.classify(cfg, cu2, sc2)
    a.compact_prompt(cu2, k2, v2, sc2, t2b)
    b.compact_prompt(cu2, k2, v2, sc2, t2b, levels_impl=True)
    _states_equal(a, b, "re-admission")


class LevelSetModel:
    """The K-level step written from the readings: sets of positions per
    level, exact rational means; returns the new sets and the case."""

    def __init__(self, W, alphas):
        self.W = W
        self.al = [Fraction(float(np.float32(x))) for x in alphas]
        self.K = len(alphas)

    def cls(self, mean, Np):
        for lv in range(self.K - 1):
            if mean * Np > self.al[lv]:
                return lv
        return self.K - 1 if mean * Np >= self.al[-1] else None

    def step(self, levels, sums, N):
        levels = [set(x) for x in levels]
        Np = N + 1
        mean = lambda p: Fraction(float(sums[p])) / (N - 1 - p)
        levels[0].add(N)
        tc = N - self.W
        if tc < 0:
            return levels, ("none",)
        assert tc in levels[0]
        c = self.cls(mean(tc), Np)
        if c == 0:
            v = min((p for p in levels[0] if p <= tc), key=lambda p: (mean(p), p))
            cv = self.cls(mean(v), Np)
            if cv != 0:
                levels[0].remove(v)
                if cv is not None:
                    levels[cv].add(v)
            return levels, (0, cv)
        levels[0].remove(tc)
        if c is None:
            return levels, (None,)
        v = min(list(levels[c]) + [tc], key=lambda p: (mean(p), p))
        levels[c].add(tc)
        cv = self.cls(mean(v), Np)
        if v != tc and cv != c:
            levels[c].remove(v)
            if cv is not None:
                levels[cv].add(v)
            return levels, (c, cv)
        return levels, (c, "keep")


def _level_sets(st, b, h):
    levels = [set() for _ in range(st.K)]
    sums = {}
    for lv, s, rec in st.unit_tokens(b, h):
        levels[lv].add(rec["pos"])
        sums[rec["pos"]] = rec["score"]
    return levels, sums


@pytest.mark.parametrize("K,per_head", [(3, False), (4, False), (3, True)])
def test_levels_step_matches_set_model(orc, K, per_head):
    rng = np.random.default_rng({(3, False): 0, (4, False): 0, (3, True): 1}[K, per_head])
    d, H, G, B, W = 64, 2, 2, 2, 6
    cfg = _cfg3() if K == 3 else _cfg4()
    ah, al = [cfg["alpha_h"]] * H, [cfg["alpha_l"]] * H
    if per_head:
        ah, al = [1.0, 1.1], [0.75, 0.7]
        cfg.update(alpha_h_head=ah, alpha_l_head=al, alpha_h=9.0, alpha_l=0.0)
    models = [LevelSetModel(W, [ah[h]] + list(cfg["alpha_mid"][:K - 2]) + [al[h]]) for h in range(H)]
    lens = np.array([40, 3])
    cu, k, v, sc, scale = _prompt_inputs(rng, H, d, lens)
    tiers, counts = orc.classify(cfg, cu, sc)
    st = orc.State(cfg, batch=B, num_pages=300)
    st.compact_prompt(cu, k, v, sc, tiers)
    assert np.array_equal(st.tier_state[..., :K], counts)
    check_pool_invariants(orc, st)
    seq = lens.astype(np.int32).copy()
    cases = {}
    for step in range(300):
        expect = {}
        for b in range(B):
            for h in range(H):
                levels, sums = _level_sets(st, b, h)
                expect[b, h] = models[h].step(levels, sums, int(seq[b]))
        state0 = st.tier_state.copy()
        end0 = int(st.ptr[1])
        kn = (rng.standard_normal((B, H, d)) * scale).astype(np.float16).view(np.uint16)
        vn = (rng.standard_normal((B, H, d)) * scale).astype(np.float16).view(np.uint16)
        st.compact_step(seq, kn, vn)
        assert st.status[0] == 0
        assert int(st.ptr[1]) == end0  # no reclamation
        grow = st.tier_state[..., K:].sum(-1) - state0[..., K:].sum(-1)
        assert np.all((grow >= 0) & (grow <= 1))  # at most one new page per unit
        for b in range(B):
            for h in range(H):
                levels, _ = _level_sets(st, b, h)
                want, case = expect[b, h]
                assert levels == want, (step, b, h, case)
                cases[case] = cases.get(case, 0) + 1
        check_pool_invariants(orc, st)
        q = (rng.standard_normal((B, H * G, d)) * 3).astype(np.float16).view(np.uint16)
        st.decode_attn(q, seq, update_scores=True)
        seq += 1
    # t_c kept in level 0, pruned, kept in the last level; level-0 victims to
    # every lower level and pruned; level-1 victims moving further down and pruned
    want = {(0, 0), (None,), (K - 1, "keep")} | {(0, lv) for lv in range(1, K)} | {(0, None), (1, None)}
    assert want <= set(cases), sorted(cases, key=str)
    assert any(c[0] == 1 and isinstance(c[1], int) and c[1] >= 2 for c in cases), sorted(cases, key=str)


def test_levels_classify_worked_boundaries(orc):
    # K = 3 at N = 8, alphas (1, 1/2, 1/4): s N = 1 is not above alpha_0 ->
    # level 1; s N = 1/2 is not above alpha_1 -> level 2; s N = 1/4 meets
    # alpha_2 -> level 2; s N = 1/8 -> pruned; the last W = 2 tokens are level 0
    cfg = _cfg3(num_kv_heads=1, alpha_h=1.0, alpha_mid=[0.5], alpha_l=0.25, window=2)
    N = 8
    s = np.array([[2.0, 1.0, 0.75, 0.5, 0.25, 0.125, 0.0, 0.0]], np.float32) / N
    tiers, counts = orc.classify(cfg, [0, N], s)
    level = [0, 1, 1, 2, 2, None, 0, 0]
    assert tiers[0].tolist() == [0 if lv is None else 3 - lv for lv in level]
    assert counts[0, 0].tolist() == [3, 2, 2]
    # the alpha/i rule uses i = position + 1 instead of N
    cfg_i = dict(cfg, prompt_rule=1, window=0)
    tiers_i, _ = orc.classify(cfg_i, [0, N], np.full((1, N), 0.3, np.float32))
    # 0.3 i > 1 for i >= 4; > 0.5 for i = 2, 3; >= 0.25 for i = 1
    assert tiers_i[0].tolist() == [1, 2, 2, 3, 3, 3, 3, 3]


def _place(orc, cfg, counts_per_level, N, P=40):
    """Prompt compaction of one unit whose tokens (first positions) take the
    given level counts; returns the state."""
    K = len(counts_per_level)
    cfg = dict(cfg, num_kv_heads=1, window=0)
    d = cfg["head_dim"]
    tiers = np.zeros((1, N), np.uint8)
    p = 0
    for lv, n in enumerate(counts_per_level):
        tiers[0, p:p + n] = K - lv
        p += n
    st = orc.State(cfg, 1, P)
    z = np.zeros((N, 1, d), np.uint16)
    st.compact_prompt([0, N], z, z, np.zeros((1, N), np.float32), tiers)
    assert st.status[0] == 0
    return st


def test_levels_prompt_block_placement_worked_examples(orc):
    cfg = _cfg3()
    Lr = orc.table_len(cfg) // 2
    # N = 100: block of 7 pages b0..b6; levels 0 and 2 take b0, b1 and b2, b3
    # from the left, level 1 takes b6 from the right; b4, b5 return to the list
    st = _place(orc, cfg, [20, 30, 40], 100)
    row = st.page_table[0, 0]
    assert row[0] == 0 and row[1] == 1 and row[Lr + 0] == 2 and row[Lr + 1] == 3 and row[Lr - 1] == 6
    assert st.free_list[40 % 40] == 4 and st.free_list[41 % 40] == 5  # appended at the old end
    assert int(st.ptr[0]) == 7 and int(st.ptr[1]) == 42
    assert st.tier_state[0, 0].tolist() == [20, 30, 40, 2, 1, 2]
    check_pool_invariants(orc, st)
    # N = 17: block of 2 pages; levels 0 and 2 fill it from the left, level 1
    # gets the extra page taken after the block
    st = _place(orc, cfg, [1, 8, 8], 17)
    row = st.page_table[0, 0]
    assert row[0] == 0 and row[Lr] == 1 and row[Lr - 1] == 2 and int(st.ptr[0]) == 3
    check_pool_invariants(orc, st)
    # K = 4, N = 33: block of 3; levels 0, 2, 3 (one page each) fill it from
    # the left; level 1's two pages are extras, innermost (page 1) first
    cfg4 = _cfg4()
    Lr4 = orc.table_len(cfg4) // 2
    st = _place(orc, cfg4, [1, 40, 1, 1], 43)
    row = st.page_table[0, 0]
    assert row[0] == 0 and row[Lr4] == 1 and row[2 * Lr4 - 1] == 2
    assert row[Lr4 - 2] == 3 and row[Lr4 - 1] == 4 and int(st.ptr[0]) == 5
    check_pool_invariants(orc, st)
    # release: row by row, left level left to right then right level right to left
    st.release([1])
    assert st.free_list[40 % 40:40 % 40 + 0].size == 0
    end = int(st.ptr[1])
    got = [int(st.free_list[i % 40]) for i in range(end - 5, end)]
    assert got == [0, 4, 3, 1, 2]  # level 0; level 1 pages 0, 1; level 2; level 3
    check_pool_invariants(orc, st)


def test_levels_attention_on_a_lossless_grid(orc):
    # Every K and V vector takes values z + s c, c = 0 .. 2^b - 1 on its own
    # level's grid (s a power of two, z a multiple of s, min and max present),
    # so the codec's scale and zero are s and z exactly and dequantization
    # returns the inputs:
    # the oracle's attention equals softmax attention over the retained
    # tokens computed here from the inputs.
    rng = np.random.default_rng(5)
    cfg = _cfg4(num_kv_heads=1, gqa_group=3, window=4)
    d, G, K = 64, 3, 4
    bits = [(8, 8), (8, 4), (4, 4), (4, 2)]
    N = 120
    sc = (rng.random((1, N)) ** 3).astype(np.float32)
    sc /= sc.sum() / 3
    tiers, _ = orc.classify(cfg, [0, N], sc)
    kx = np.zeros((N, d), np.float32)
    vx = np.zeros((N, d), np.float32)
    for t in range(N):
        lv = K - int(tiers[0, t]) if tiers[0, t] else 0
        for x, b in ((kx, bits[lv][0]), (vx, bits[lv][1])):
            s = 2.0 ** -int(rng.integers(2, 5))
            z = s * int(rng.integers(-300, 300))  # every grid value s (m + c), |m + c| < 2048: exact in fp16
            codes = rng.integers(0, 2 ** b, d)
            codes[0], codes[1] = 0, 2 ** b - 1  # min and max present
            x[t] = (np.float32(z) + np.float32(s) * codes.astype(np.float32))
    k16 = kx.astype(np.float16)
    v16 = vx.astype(np.float16)
    assert np.array_equal(k16.astype(np.float32), kx) and np.array_equal(v16.astype(np.float32), vx)
    st = orc.State(cfg, 1, 40)
    st.compact_prompt([0, N], k16.view(np.uint16).reshape(N, 1, d), v16.view(np.uint16).reshape(N, 1, d), sc,
                      tiers)
    q = rng.standard_normal((1, G, d)).astype(np.float16)
    out = st.decode_attn(q.view(np.uint16), np.array([N], np.int32))
    keep = tiers[0] > 0
    kk, vv = kx[keep].astype(np.float64), vx[keep].astype(np.float64)
    for g in range(G):
        x = kk @ q[0, g].astype(np.float64) / np.sqrt(d)
        p = np.exp(x - x.max())
        p /= p.sum()
        assert np.allclose(out[0, g], p @ vv, rtol=0, atol=1e-5), g
