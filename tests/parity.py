"""Helpers for GPU-vs-oracle parity tests: run the same seeded inputs through
the C-ABI library (device) and the oracle (host) and compare."""
from __future__ import annotations

import numpy as np
import torch

ATOL, RTOL = 2e-3, 1e-3          # attention outputs: |gpu - ref| <= ATOL + RTOL |ref|
SCORE_ATOL, SCORE_RTOL = 1e-5, 1e-4   # score sums after the fp32 update


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def gpu_pages(g) -> np.ndarray:
    return np_(g.pool.pages.view(g.pool.num_pages, -1))


def live_pages(page_table: np.ndarray) -> list:
    return sorted({int(x) for x in page_table.ravel() if x >= 0})


def plan_record_span(cfg) -> tuple:
    """Bytes after the last segment of a high page that the library uses for
    its private plan record (the oracle leaves them zero); none for a tier
    codec variant, which keeps no plan records."""
    from oracle import HI, tier_layout
    _, seg = tier_layout(cfg, HI)
    if any(cfg.get(k, 0) for k in ("hi_k_bits", "hi_v_bits", "lo_k_bits", "lo_v_bits")):
        return int(seg[6]), 0
    return int(seg[6]), 64


def first_pages(page_table: np.ndarray) -> set:
    """Page ids at table entry 0 (a unit's first high page)."""
    return {int(x) for x in page_table[..., 0].ravel() if x >= 0}


def masked(page: np.ndarray, cfg) -> np.ndarray:
    off, n = plan_record_span(cfg)
    q = page.copy()
    q[off:off + n] = 0
    return q


def assert_state_equal(g, st, pages=True, what=""):
    """Bit-exact comparison of the whole compaction state."""
    pt = np_(g.page_table)
    assert np.array_equal(pt, st.page_table), f"{what}: page tables differ"
    assert np.array_equal(np_(g.tier_state), st.tier_state), f"{what}: tier state differs"
    assert np.array_equal(np_(g.pool.free_list), st.free_list), f"{what}: free lists differ"
    assert np.array_equal(np_(g.pool.ptr).view(np.uint64), st.ptr), f"{what}: pointers differ"
    assert int(np_(g.pool.status)[0]) == int(st.status[0]), \
        f"{what}: status {int(np_(g.pool.status)[0])} vs {int(st.status[0])}"
    if pages:
        live = live_pages(st.page_table)
        gp = gpu_pages(g)
        first = first_pages(st.page_table)
        bad = [p for p in live
               if not np.array_equal(masked(gp[p], st.cfg) if p in first else gp[p], st.pages[p])]
        assert not bad, f"{what}: {len(bad)} of {len(live)} live pages differ, first {bad[:5]}"


def assert_attn_close(out_g, out_o, what=""):
    out_g = np_(out_g) if isinstance(out_g, torch.Tensor) else out_g
    err = np.abs(out_g - out_o)
    tol = ATOL + RTOL * np.abs(out_o)
    assert np.all(np.isfinite(out_g)), f"{what}: non-finite outputs"
    assert np.all(err <= tol), f"{what}: attention max err {err.max():.3e} (worst ratio {(err / tol).max():.2f})"
    return float(err.max())


def assert_scores_close(g, st, what=""):
    """Score sums of every live slot within tolerance; everything else bit-exact."""
    gp = gpu_pages(g)
    live = live_pages(st.page_table)
    from oracle import level_layout, num_levels
    cfg = st.cfg
    first = first_pages(st.page_table)
    for p in live:
        a, b = gp[p].copy(), st.pages[p].copy()
        if p in first:
            a = masked(a, cfg)
        if np.array_equal(a, b):
            continue
        for lv in range(max(num_levels(cfg), 2)):  # the page's level: the one whose score segment explains it
            _, seg = level_layout(cfg, lv)
            sa = a[seg[4]:seg[5]].view(np.float32)
            sb = b[seg[4]:seg[5]].view(np.float32)
            a2, b2 = a.copy(), b.copy()
            a2[seg[4]:seg[5]] = 0
            b2[seg[4]:seg[5]] = 0
            if np.array_equal(a2, b2):
                assert np.all(np.abs(sa - sb) <= SCORE_ATOL + SCORE_RTOL * np.abs(sb)), \
                    f"{what}: page {p} score sums differ beyond tolerance"
                break
        else:
            raise AssertionError(f"{what}: page {p} differs outside the score segment")


def resync_scores(g, st):
    """Copy the oracle's page bytes (incl. score sums) to the device so later
    steps start from identical state (fp32 sums are tolerance-equal only)."""
    live = live_pages(st.page_table)
    pages = g.pool.pages.view(g.pool.num_pages, -1)
    idx = torch.tensor(live, dtype=torch.int64, device=pages.device)
    pages[idx] = torch.from_numpy(st.pages[live]).to(pages.device)
    # pages written from outside the library: plans made from the old scores
    # no longer apply (the next decode step runs the plan kernel)
    g.chain = 0
    torch.cuda.synchronize()


def _unit_pages(st):
    """(high page ids, low page ids, first-page ids) of the oracle state's units."""
    pt, ts = st.page_table, st.tier_state
    L = pt.shape[-1]
    hi, lo, first = [], [], set()
    for b in range(pt.shape[0]):
        for h in range(pt.shape[1]):
            ph, pl = int(ts[b, h, 2]), int(ts[b, h, 3])
            hi += [int(x) for x in pt[b, h, :ph]]
            lo += [int(x) for x in pt[b, h, L - pl:]]
            if ph:
                first.add(int(pt[b, h, 0]))
    return np.array(hi, np.int64), np.array(lo, np.int64), first


def compare_pages_scores_tol(g, st, what=""):
    """Every live page byte-identical outside its tier's score segment (and
    the plan-record span of a unit's first page), score sums within
    SCORE_ATOL + SCORE_RTOL |ref|.  Vectorized over pages."""
    from oracle import tier_layout, HI, LO
    hi, lo, first = _unit_pages(st)
    pages = g.pool.pages.view(g.pool.num_pages, -1)
    off, n = plan_record_span(st.cfg)
    worst = 0.0
    for ids, tier in ((hi, HI), (lo, LO)):
        if ids.size == 0:
            continue
        _, seg = tier_layout(st.cfg, tier)
        a = np_(pages.index_select(0, torch.from_numpy(ids).to(pages.device)))
        b = st.pages[ids]
        isf = np.array([int(x) in first for x in ids])
        a[isf, off:off + n] = 0
        keep = np.ones(a.shape[1], bool)
        keep[seg[4]:seg[5]] = False
        bad = np.flatnonzero(~np.all(a[:, keep] == b[:, keep], axis=1))
        assert bad.size == 0, f"{what}: {bad.size} of {ids.size} pages differ outside the score segment, " \
                              f"first page ids {ids[bad[:5]].tolist()}"
        sa = np.ascontiguousarray(a[:, seg[4]:seg[5]]).view(np.float32)
        sb = np.ascontiguousarray(b[:, seg[4]:seg[5]]).view(np.float32)
        err = np.abs(sa.astype(np.float64) - sb)
        tol = SCORE_ATOL + SCORE_RTOL * np.abs(sb.astype(np.float64))
        assert np.all(err <= tol), f"{what}: score sums differ beyond tolerance (worst ratio {(err / tol).max():.2f})"
        worst = max(worst, float((err / tol).max()))
    return worst


def sync_scores_to_oracle(g, st):
    """Copy the device's score segments into the oracle's pages (the other
    direction of resync_scores): the device's plans for the next step stay
    valid, and both sides then decide the next step from the same sums."""
    from oracle import tier_layout, HI, LO
    hi, lo, _ = _unit_pages(st)
    pages = g.pool.pages.view(g.pool.num_pages, -1)
    for ids, tier in ((hi, HI), (lo, LO)):
        if ids.size == 0:
            continue
        _, seg = tier_layout(st.cfg, tier)
        a = np_(pages.index_select(0, torch.from_numpy(ids).to(pages.device)))
        st.pages[ids, seg[4]:seg[5]] = a[:, seg[4]:seg[5]]
