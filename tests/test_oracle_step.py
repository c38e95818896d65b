"""Pins of the oracle's generation step (CPU only).

Source: DiffKV notes, "KV compression policy" (generation phase: one token
is compressed per step, the window's oldest token t_c is classified, then
the least important token t_v of the receiving tier may be requantized or
pruned; algorithm flow against alpha/N) and "Memory management" (generation
workflow: a head allocates only when a page is full, at most one page per
step, no reclamation until the request completes).

The policy is re-derived here as a second, set-based model (positions per
tier, exact rational means, no slots or pages) and run against the oracle for
hundreds of steps with real score updates in between.
"""
from fractions import Fraction

import numpy as np
import pytest

from tests.invariants import check_pool_invariants


class SetModel:
    HI, LO, PRUNE = "hi", "lo", "prune"

    def __init__(self, W, alpha_h, alpha_l, lo_enabled):
        self.W = W
        self.ah = Fraction(float(np.float32(alpha_h)))
        self.al = Fraction(float(np.float32(alpha_l)))
        self.lo_enabled = lo_enabled

    def cls(self, mean, Np):
        th_h, th_l = self.ah / Np, self.al / Np
        if self.lo_enabled:
            if mean > th_h:
                return self.HI
            return self.LO if mean >= th_l else self.PRUNE
        return self.HI if mean >= th_l else self.PRUNE

    def step(self, hi, lo, sums, N):
        """hi, lo: sets of positions; sums: pos -> fp32 score sum. Returns new sets."""
        hi, lo = set(hi), set(lo)
        Np = N + 1
        mean = lambda p: Fraction(float(sums[p])) / (N - 1 - p)
        hi.add(N)
        tc = N - self.W
        cases = None
        if tc >= 0:
            assert tc in hi
            c = self.cls(mean(tc), Np)
            if c == self.HI:
                v = min((p for p in hi if p <= tc), key=lambda p: (mean(p), p))
                cv = self.cls(mean(v), Np)
                if cv == self.LO:
                    hi.remove(v)
                    lo.add(v)
                elif cv == self.PRUNE:
                    hi.remove(v)
                cases = "hi/" + cv
            elif c == self.LO:
                hi.remove(tc)
                v = min(list(lo) + [tc], key=lambda p: (mean(p), p))
                lo.add(tc)
                pruned = v != tc and self.cls(mean(v), Np) == self.PRUNE
                if pruned:
                    lo.remove(v)
                cases = "lo/" + ("prune" if pruned else "keep")
            else:
                hi.remove(tc)
                cases = "prune"
        return hi, lo, cases


def _sets(st, b, h, orc):
    hi, lo, sums = set(), set(), {}
    for t, s, rec in st.unit_tokens(b, h):
        (hi if t == orc.HI else lo).add(rec["pos"])
        sums[rec["pos"]] = rec["score"]
    return hi, lo, sums


@pytest.mark.parametrize("lo_enabled,per_head,codec", [(1, False, None), (0, False, None), (1, True, None),
                                                      (1, False, (4, 8, 2, 4)), (1, False, (8, 2, 4, 1))])
def test_step_matches_set_model(orc, lo_enabled, per_head, codec):
    # per_head: each KV head classifies against its own (alpha_h, alpha_l)
    # ("KV compression policy", extensibility paragraph); the set model runs
    # one policy per head with that head's pair
    rng = np.random.default_rng(100 + lo_enabled + 7 * per_head + (sum(codec) if codec else 0))
    d, H, G, B, W = 64, 2, 2, 2, 6
    cfg = dict(head_dim=d, num_kv_heads=H, gqa_group=G, max_seq_len=700, window=W,
               alpha_h=1.0, alpha_l=0.3, lo_enabled=lo_enabled)
    if codec is not None:  # tier codec variant (the policy does not depend on it)
        cfg.update(hi_k_bits=codec[0], hi_v_bits=codec[1], lo_k_bits=codec[2], lo_v_bits=codec[3])
    ah, al = [1.0] * H, [0.3] * H
    if per_head:
        ah, al = [1.0, 2.5], [0.3, 0.6]
        cfg.update(alpha_h_head=ah, alpha_l_head=al, alpha_h=9.0, alpha_l=9.0)
    lens = np.array([40, 3])         # the second prompt is shorter than the window
    cu = np.concatenate([[0], np.cumsum(lens)])
    total = int(cu[-1])
    scale = np.ones(d, np.float32)
    scale[[3, 17]] = 8.0
    k = (rng.standard_normal((total, H, d)) * scale).astype(np.float16).view(np.uint16)
    v = (rng.standard_normal((total, H, d)) * scale).astype(np.float16).view(np.uint16)
    sc = (rng.random((H, total)) ** 4).astype(np.float32)
    sc /= sc.sum(1, keepdims=True) / 4
    tiers, _ = orc.classify(cfg, cu, sc)
    st = orc.State(cfg, batch=B, num_pages=200)
    st.compact_prompt(cu, k, v, sc, tiers)
    models = [SetModel(W, ah[h], al[h], lo_enabled) for h in range(H)]
    seq = lens.astype(np.int32).copy()
    gone = [[set() for _ in range(H)] for _ in range(B)]
    cases = {}
    for step in range(400):
        expect = {}
        for b in range(B):
            for h in range(H):
                hi, lo, sums = _sets(st, b, h, orc)
                expect[b, h] = models[h].step(hi, lo, sums, int(seq[b]))
        state0 = st.tier_state.copy()
        end0 = int(st.ptr[1])
        kn = (rng.standard_normal((B, H, d)) * scale).astype(np.float16).view(np.uint16)
        vn = (rng.standard_normal((B, H, d)) * scale).astype(np.float16).view(np.uint16)
        st.compact_step(seq, kn, vn)
        assert st.status[0] == 0
        assert int(st.ptr[1]) == end0                       # no reclamation
        pages0 = state0[..., 2] + state0[..., 3]
        pages1 = st.tier_state[..., 2] + st.tier_state[..., 3]
        assert np.all((pages1 - pages0 >= 0) & (pages1 - pages0 <= 1))
        assert np.all(st.tier_state[..., :2] >= state0[..., :2])   # tiers never shrink
        for b in range(B):
            for h in range(H):
                hi, lo, _ = _sets(st, b, h, orc)
                ehi, elo, case = expect[b, h]
                assert hi == ehi and lo == elo, (step, b, h, case)
                cases[case] = cases.get(case, 0) + 1
                N1 = int(seq[b]) + 1
                assert set(range(max(0, N1 - W), N1)) <= hi         # window always high
                old_hi, old_lo, _ = _sets_prev[b][h] if step else (set(), set(), None)
                assert not (hi & gone[b][h]) and not (lo & gone[b][h])
                assert not (hi & old_lo)                              # no re-promotion
                gone[b][h] |= (old_hi | old_lo) - (hi | lo)
        _sets_prev = [[_sets(st, b, h, orc) for h in range(H)] for b in range(B)]
        check_pool_invariants(orc, st)
        q = rng.standard_normal((B, H * G, d)).astype(np.float16).view(np.uint16)
        st.decode_attn(q, seq, update_scores=True)
        seq += 1
    # every branch of the policy was taken
    want = {"hi/hi", "prune"} | ({"hi/lo", "lo/keep", "lo/prune"} if lo_enabled else {"hi/prune"})
    assert want <= set(cases), cases


def test_step_page_growth_and_exhaustion(orc):
    # A unit whose high tier is full allocates exactly one page; with an
    # empty free list the whole call commits nothing.
    rng = np.random.default_rng(3)
    d = 64
    cfg = dict(head_dim=d, num_kv_heads=1, gqa_group=1, max_seq_len=100, window=64,
               alpha_h=1.0, alpha_l=0.2)
    N = 32                                    # 32 window tokens -> 2 full hi pages
    k = rng.standard_normal((N, 1, d)).astype(np.float16).view(np.uint16)
    st = orc.State(cfg, batch=1, num_pages=2)
    tiers, _ = orc.classify(cfg, [0, N], np.zeros((1, N), np.float32))
    st.compact_prompt([0, N], k, k, np.zeros((1, N), np.float32), tiers)
    assert st.tier_state[0, 0].tolist() == [32, 0, 2, 0] and int(st.ptr[1] - st.ptr[0]) == 0
    before = st.copy()
    st.compact_step([N], k[:1, :, :].reshape(1, 1, d), k[:1].reshape(1, 1, d))
    assert st.status[0] == orc.ST_POOL_EXHAUSTED
    assert np.array_equal(st.pages, before.pages) and np.array_equal(st.tier_state, before.tier_state)
    st2 = orc.State(cfg, batch=1, num_pages=3)
    st2.compact_prompt([0, N], k, k, np.zeros((1, N), np.float32), tiers)
    st2.compact_step([N], k[:1].reshape(1, 1, d), k[:1].reshape(1, 1, d))
    assert st2.status[0] == 0 and st2.tier_state[0, 0].tolist() == [33, 0, 3, 0]
    assert st2.page_table[0, 0, 2] == 2
    check_pool_invariants(orc, st2)


def test_step_rejects_overflow_and_small_window(orc):
    d = 64
    cfg = dict(head_dim=d, num_kv_heads=1, gqa_group=1, max_seq_len=32, window=8,
               alpha_h=1.0, alpha_l=0.2)
    rng = np.random.default_rng(2)
    N = 32
    k = rng.standard_normal((N, 1, d)).astype(np.float16).view(np.uint16)
    st = orc.State(cfg, batch=1, num_pages=8)
    tiers, _ = orc.classify(cfg, [0, N], np.zeros((1, N), np.float32))
    st.compact_prompt([0, N], k, k, np.zeros((1, N), np.float32), tiers)
    st.compact_step([N], k[:1].reshape(1, 1, d), k[:1].reshape(1, 1, d))
    assert st.status[0] & orc.ST_TABLE_OVERFLOW
    with pytest.raises(ValueError):
        orc.State(dict(cfg, window=1), batch=1, num_pages=8).compact_step(
            [4], k[:1].reshape(1, 1, d), k[:1].reshape(1, 1, d))
