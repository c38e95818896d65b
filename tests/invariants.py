"""Allocator invariants checked on any host copy of the compaction state.

From the circular free page list and bidirectional page table of the DiffKV
notes ("Memory management"): every page id is either in the free region of
the list or in exactly one table row, never both and never twice; the free
region is [start, end) of the monotonic counters; hi ids fill a prefix of a
row and lo ids a suffix (with K levels, each row holds two levels that way).
"""
import numpy as np


def check_pool_invariants(orc, st, T_h: int = 16, T_l: int = 32):
    P = int(st.num_pages)
    start, end = int(st.ptr[0]), int(st.ptr[1])
    assert 0 <= end - start <= P, (start, end, P)
    seen = np.zeros(P, np.int32)
    for i in range(end - start):
        seen[st.free_list[(start + i) % P]] += 1
    B, H, L = st.page_table.shape
    K = st.tier_state.shape[2] // 2
    if K > 2:  # K levels: row r holds level 2r from the left, 2r+1 from the right
        R = (K + 1) // 2
        Lr = L // R
        for b in range(B):
            for h in range(H):
                s = [int(x) for x in st.tier_state[b, h]]
                for lv in range(K):
                    T = T_h if lv == 0 else T_l
                    assert s[K + lv] == -(-s[lv] // T), (b, h, s)
                for r in range(R):
                    row = st.page_table[b, h, r * Lr:(r + 1) * Lr]
                    a = s[K + 2 * r]
                    c = s[K + 2 * r + 1] if 2 * r + 1 < K else 0
                    assert a + c <= Lr
                    used = list(row[:a]) + [row[Lr - 1 - j] for j in range(c)]
                    assert np.all(row[a:Lr - c] == -1), (b, h, r, row)
                    for pid in used:
                        assert 0 <= pid < P
                        seen[pid] += 1
        assert np.all(seen == 1), np.flatnonzero(seen != 1)[:10]
        return
    for b in range(B):
        for h in range(H):
            n_hi, n_lo, ph, pl = (int(x) for x in st.tier_state[b, h])
            assert ph == -(-n_hi // T_h) and pl == -(-n_lo // T_l), (b, h, n_hi, n_lo, ph, pl)
            assert ph + pl <= L
            row = st.page_table[b, h]
            used = list(row[:ph]) + [row[L - 1 - j] for j in range(pl)]
            rest = np.concatenate([row[ph:L - pl]]) if L - pl > ph else np.zeros(0, np.int32)
            assert np.all(rest == -1), (b, h, row)
            for pid in used:
                assert 0 <= pid < P
                seen[pid] += 1
    assert np.all(seen == 1), np.flatnonzero(seen != 1)[:10]
