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
    its private plan record (the oracle leaves them zero)."""
    from oracle import HI, tier_layout
    _, seg = tier_layout(cfg, HI)
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
    from oracle import tier_layout, HI, LO
    cfg = st.cfg
    first = first_pages(st.page_table)
    for p in live:
        a, b = gp[p].copy(), st.pages[p].copy()
        if p in first:
            a = masked(a, cfg)
        if np.array_equal(a, b):
            continue
        for t in (HI, LO):
            _, seg = tier_layout(cfg, t)
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
