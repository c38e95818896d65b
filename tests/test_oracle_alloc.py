"""Pins of the oracle's allocator, tables, packing and release (CPU only).

Sources: DiffKV notes, "Memory management": circular free page list (one
contiguous list, allocation pointer start, reclamation pointer end, both
wrapping, prefix sums give disjoint regions), bidirectional page table (hi
ids grow left to right, lo ids right to left), Fig 6 prompt workflow
(8-token request, 2-token hi pages, 4-token lo pages: pages 5-8 to head A,
9-12 to head B, pointer to 13, A keeps 1 hi + 1 lo page, B 2 hi + 1 lo,
6, 7 and 11 reclaimed), generation workflow (at most one new page per head
per step, no reclamation until the request completes).
"""
import os

import numpy as np
import pytest

from tests.invariants import check_pool_invariants


def _golden(name):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                key, *rest = line.split()
                vals[key] = [int(x) for x in rest]
    return vals


def test_fig6_worked_example_literal(orc):
    # Small pages exactly as in the figure (tests/golden/fig6_prompt_allocation.txt).
    g = _golden("fig6_prompt_allocation.txt")
    P, th, tl, N = g["pool_pages"][0], g["hi_page_tokens"][0], g["lo_page_tokens"][0], g["seq_len"][0]
    L = -(-N // th) + 1
    free_list = np.arange(P, dtype=np.int32)
    ptr = np.array([g["alloc_start"][0], P], np.uint64)
    status = np.zeros(1, np.uint32)
    table = np.full((1, 2, L), -1, np.int32)
    state = np.zeros((1, 2, 4), np.int32)
    n_hi = [g["head_A_tokens"][0], g["head_B_tokens"][0]]
    n_lo = [g["head_A_tokens"][1], g["head_B_tokens"][1]]
    orc.prompt_allocate(2, th, tl, L, [N], n_hi, n_lo, free_list, ptr, status, table, state)
    assert status[0] == 0
    assert table[0, 0].tolist() == g["table_A"]
    assert table[0, 1].tolist() == g["table_B"]
    assert int(ptr[0]) == g["alloc_pointer_after"][0]
    freed = g["reclaimed_in_order"]
    assert int(ptr[1]) == P + len(freed)
    assert free_list[[(P + i) % P for i in range(len(freed))]].tolist() == freed
    assert state.tolist() == [[[n_hi[0], n_lo[0], 1, 1], [n_hi[1], n_lo[1], 2, 1]]]


def _fig6_scaled_inputs(orc, d=128):
    # Same example with this build's 16/32-token pages: every token count x8.
    cfg = dict(head_dim=d, num_kv_heads=2, gqa_group=1, max_seq_len=64, window=0,
               alpha_h=1.0, alpha_l=0.2)
    N = 64
    tiers = np.zeros((2, N), np.uint8)
    tiers[0, :16] = orc.HI          # A: 16 hi (1 page) + 24 lo (1 page)
    tiers[0, 16:40] = orc.LO
    tiers[1, 0:17] = orc.HI         # B: 17 hi (2 pages) + 20 lo (1 page)
    tiers[1, 30:50] = orc.LO
    rng = np.random.default_rng(3)
    k = rng.standard_normal((N, 2, d)).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((N, 2, d)).astype(np.float16).view(np.uint16)
    scores = rng.random((2, N)).astype(np.float32) / N
    return cfg, N, tiers, k, v, scores


def test_fig6_worked_example_scaled_full_compaction(orc):
    cfg, N, tiers, k, v, scores = _fig6_scaled_inputs(orc)
    st = orc.State(cfg, batch=1, num_pages=16)
    st.ptr[0] = 5                     # pages 0-4 in use
    st.compact_prompt([0, N], k, v, scores, tiers)
    L = st.L
    assert L == 5
    assert st.status[0] == 0
    assert st.page_table[0, 0].tolist() == [5, -1, -1, -1, 8]
    assert st.page_table[0, 1].tolist() == [9, 10, -1, -1, 12]
    assert int(st.ptr[0]) == 13 and int(st.ptr[1]) == 16 + 3
    assert st.free_list[[0, 1, 2]].tolist() == [6, 7, 11]


def test_pack_slots_follow_position_order(orc):
    cfg, N, tiers, k, v, scores = _fig6_scaled_inputs(orc)
    st = orc.State(cfg, batch=1, num_pages=16)
    st.compact_prompt([0, N], k, v, scores, tiers)
    d = cfg["head_dim"]
    for h in range(2):
        toks = st.unit_tokens(0, h)
        hi_pos = [rec["pos"] for t, s, rec in toks if t == orc.HI]
        lo_pos = [rec["pos"] for t, s, rec in toks if t == orc.LO]
        assert hi_pos == np.flatnonzero(tiers[h] == orc.HI).tolist()
        assert lo_pos == np.flatnonzero(tiers[h] == orc.LO).tolist()
        for t, s, rec in toks:
            p = rec["pos"]
            xk = k[p, h].view(np.float16).astype(np.float32)
            xv = v[p, h].view(np.float16).astype(np.float32)
            kb, vb = (8, 4) if t == orc.HI else (4, 2)
            s_, z_, c_ = orc.quantize(xk, kb)
            assert rec["kmeta"].tolist() == [s_, z_] and np.array_equal(rec["k"], c_)
            s_, z_, c_ = orc.quantize(xv, vb)
            assert rec["vmeta"].tolist() == [s_, z_] and np.array_equal(rec["v"], c_)
            # stored score = mean x (N - 1 - p), one fp32 multiply
            assert rec["score"] == np.float32(scores[h, p]) * np.float32(N - 1 - p)
    # unused slots of allocated pages are zero
    row = st.page_table[0, 0]
    _, seg = orc.tier_layout(cfg, orc.HI)
    page = st.pages[row[0]]
    assert not page[seg[6]:].any()


def test_extra_page_when_block_is_short(orc):
    # S_max = 32: 17 hi + 15 lo tokens need 2 + 1 pages from a 2-page block
    cfg = dict(head_dim=64, num_kv_heads=1, gqa_group=1, max_seq_len=32, window=0,
               alpha_h=1.0, alpha_l=0.2)
    N = 32
    tiers = np.zeros((1, N), np.uint8)
    tiers[0, :17] = orc.HI
    tiers[0, 17:] = orc.LO
    rng = np.random.default_rng(4)
    k = rng.standard_normal((N, 1, 64)).astype(np.float16).view(np.uint16)
    st = orc.State(cfg, batch=1, num_pages=8)
    st.compact_prompt([0, N], k, k, np.zeros((1, N), np.float32), tiers)
    assert st.status[0] == 0
    assert st.page_table[0, 0].tolist() == [0, 1, 2]    # block [0, 1] hi, extra page 2 lo
    assert st.tier_state[0, 0].tolist() == [17, 15, 2, 1]
    assert int(st.ptr[0]) == 3 and int(st.ptr[1]) == 8
    check_pool_invariants(orc, st)


def test_all_or_nothing_on_exhaustion(orc):
    cfg, N, tiers, k, v, scores = _fig6_scaled_inputs(orc)
    st = orc.State(cfg, batch=1, num_pages=7)     # conservative block needs 8
    before = st.copy()
    st.compact_prompt([0, N], k, v, scores, tiers)
    assert st.status[0] == orc.ST_POOL_EXHAUSTED
    assert np.array_equal(st.page_table, before.page_table)
    assert np.array_equal(st.free_list, before.free_list)
    assert np.array_equal(st.ptr, before.ptr)
    assert np.array_equal(st.pages, before.pages)


def test_release_returns_pages_in_table_order(orc):
    cfg, N, tiers, k, v, scores = _fig6_scaled_inputs(orc)
    st = orc.State(cfg, batch=1, num_pages=16)
    st.compact_prompt([0, N], k, v, scores, tiers)
    end0 = int(st.ptr[1])
    st.release([1])
    # head A: hi [0] then lo [3]; head B: hi [4, 5] then lo [7]
    got = [int(st.free_list[(end0 + i) % 16]) for i in range(5)]
    assert got == [0, 3, 4, 5, 7]
    assert np.all(st.page_table == -1) and np.all(st.tier_state == 0)
    assert int(st.ptr[1] - st.ptr[0]) == 16
    check_pool_invariants(orc, st)


def test_table_overflow_and_bad_state(orc):
    cfg, N, tiers, k, v, scores = _fig6_scaled_inputs(orc)
    small = dict(cfg, max_seq_len=32)
    st = orc.State(small, batch=1, num_pages=16)
    st.compact_prompt([0, N], k, v, scores, tiers)
    assert st.status[0] & orc.ST_TABLE_OVERFLOW
    st = orc.State(cfg, batch=1, num_pages=32)
    st.compact_prompt([0, N], k, v, scores, tiers)
    before = st.copy()
    st.compact_prompt([0, N], k, v, scores, tiers)     # slot already holds a request
    assert st.status[0] & orc.ST_BAD_STATE
    assert np.array_equal(st.page_table, before.page_table)


def test_random_prompt_release_cycles_wrap(orc):
    # Property test: random ragged batches admitted and released many times on
    # a small pool, forcing the counters far past P (wrap-around) and
    # occasional exhaustion; the invariants hold after every call.
    rng = np.random.default_rng(11)
    d, H = 64, 3
    cfg = dict(head_dim=d, num_kv_heads=H, gqa_group=2, max_seq_len=200, window=8,
               alpha_h=1.0, alpha_l=0.2)
    P = 60
    B = 4
    st = orc.State(cfg, batch=B, num_pages=P)
    active = np.zeros(B, bool)
    exhausted = 0
    for it in range(150):
        rel = (rng.random(B) < 0.4) & active
        if rel.any():
            st.release(rel.astype(np.uint8))
            active &= ~rel
            assert st.status[0] == 0
            check_pool_invariants(orc, st)
        lens = np.where(~active & (rng.random(B) < 0.7), rng.integers(1, 200, B), 0)
        if lens.sum() == 0:
            continue
        cu = np.concatenate([[0], np.cumsum(lens)])
        total = int(cu[-1])
        sc = (rng.random((H, total)) ** 3 / 20).astype(np.float32)
        tiers, counts = orc.classify(cfg, cu, sc)
        kv = rng.standard_normal((total, H, d)).astype(np.float16).view(np.uint16)
        before = st.copy()
        st.compact_prompt(cu, kv, kv, sc, tiers)
        if st.status[0]:
            assert st.status[0] == orc.ST_POOL_EXHAUSTED
            exhausted += 1
            assert np.array_equal(st.page_table, before.page_table)
            assert np.array_equal(st.ptr, before.ptr)
            st.status[0] = 0
        else:
            active |= lens > 0
            for b in np.flatnonzero(lens > 0):
                for h in range(H):
                    assert st.tier_state[b, h, :2].tolist() == counts[b, h].tolist()
        check_pool_invariants(orc, st)
    assert int(st.ptr[0]) > 3 * P      # the counters wrapped several times
    assert exhausted > 0


@pytest.mark.parametrize("bad_id", [-1, 16])
def test_release_rejects_page_ids_outside_the_pool(orc, bad_id):
    # A table entry outside [0, P) in a released unit's used range would put
    # a foreign id on the free list: the call sets BAD_STATE and commits
    # nothing (other released units included).
    cfg, N, tiers, k, v, scores = _fig6_scaled_inputs(orc)
    st = orc.State(cfg, batch=1, num_pages=16)
    st.compact_prompt([0, N], k, v, scores, tiers)
    L = st.page_table.shape[-1]
    st.page_table[0, 1, L - 1] = bad_id         # head B's first low page
    before = st.copy()
    st.release([1])
    assert st.status[0] == orc.ST_BAD_STATE
    assert np.array_equal(st.page_table, before.page_table)
    assert np.array_equal(st.tier_state, before.tier_state)
    assert np.array_equal(st.free_list, before.free_list)
    assert np.array_equal(st.ptr, before.ptr)
