"""GPU parity at the workloads' full sizes, in the launch configuration
bench.py times (one split per unit at >= 256 units, several below).

* Llama3-8B-shaped layer (B32, 4096 tokens): the oracle runs the whole
  batch; state, every live page and the attention are compared as in the
  small tests.
* Long context, churn and the high-GQA stress cases: the device runs the
  whole batch; the oracle runs a sub-batch of sampled requests through the
  same calls.  Page ids depend on the other requests, so what is compared is
  what does not: tier counts, page counts and every page's bytes pairwise in
  table order (bit-exact; score sums within tolerance after an update), and
  the attention rows of the sampled requests.  The full device pool is
  checked for the allocator invariants (each page id exactly once in the free
  region or in one table row, hi prefix / lo suffix rows).
"""
import numpy as np
import pytest
import torch

from tests.parity import (SCORE_ATOL, SCORE_RTOL, assert_attn_close, assert_state_equal, masked, np_,
                          resync_scores)

pytestmark = pytest.mark.gpu

dev = torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dk():
    import compressed_paged_attention_amd as dk
    dk.lib()
    return dk


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.lib()
    return oracle


def _free_gpu():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def check_device_pool(g, T_h=16, T_l=32):
    """Allocator invariants on the device state, at any size."""
    P = int(g.pool.num_pages)
    ptr = np_(g.pool.ptr).view(np.uint64)
    start, end = int(ptr[0]), int(ptr[1])
    assert 0 <= end - start <= P, (start, end, P)
    fl = np_(g.pool.free_list)
    s0 = start % P
    n = end - start
    free_ids = np.concatenate([fl[s0:min(P, s0 + n)], fl[:max(0, s0 + n - P)]])
    ts = np_(g.tier_state).reshape(-1, 4).astype(np.int64)
    pt = np_(g.page_table)
    L = pt.shape[-1]
    rows = pt.reshape(-1, L)
    assert np.all(ts[:, 2] == -(-ts[:, 0] // T_h)) and np.all(ts[:, 3] == -(-ts[:, 1] // T_l))
    j = np.arange(L)[None, :]
    used_mask = (j < ts[:, 2:3]) | (j >= L - ts[:, 3:4])
    assert np.all(rows[~used_mask] == -1), "entries outside the hi prefix / lo suffix"
    live = rows[used_mask]
    assert live.size == 0 or (live.min() >= 0 and live.max() < P)
    counts = np.bincount(np.concatenate([free_ids.astype(np.int64), live.astype(np.int64)]), minlength=P)
    assert counts.size == P and np.all(counts == 1), \
        f"{int((counts != 1).sum())} page ids not present exactly once"


def unit_page_pairs(g_pt, g_ts, o_pt, o_ts, gb, ob, H, L):
    """(device page id, oracle page id, is_hi, is_first) for every page of the sampled
    request's units, in table order; tier state must match."""
    pairs = []
    for h in range(H):
        assert np.array_equal(g_ts[gb, h], o_ts[ob, h]), f"request {gb} head {h}: tier state differs"
        ph, pl = int(o_ts[ob, h, 2]), int(o_ts[ob, h, 3])
        for j in range(ph):
            pairs.append((int(g_pt[gb, h, j]), int(o_pt[ob, h, j]), True, j == 0))
        for j in range(pl):
            pairs.append((int(g_pt[gb, h, L - 1 - j]), int(o_pt[ob, h, L - 1 - j]), False, False))
    return pairs


def compare_sampled(g, o, orc, cfg, sample, scores_exact, what):
    """Pairwise page bytes of the sampled requests (device request sample[i]
    is oracle request i)."""
    H = int(cfg["num_kv_heads"])
    g_pt, g_ts = np_(g.page_table), np_(g.tier_state)
    L = g_pt.shape[-1]
    pairs = []
    for ob, gb in enumerate(sample):
        pairs += unit_page_pairs(g_pt, g_ts, o.page_table, o.tier_state, gb, ob, H, L)
    if not pairs:
        return pairs
    gid = torch.tensor([p[0] for p in pairs], dtype=torch.int64, device=dev)
    gp = np_(g.pool.pages.view(g.pool.num_pages, -1).index_select(0, gid))
    op = o.pages[[p[1] for p in pairs]]
    _, seg_h = orc.tier_layout(cfg, orc.HI)
    _, seg_l = orc.tier_layout(cfg, orc.LO)
    for i, (_, _, hi, first) in enumerate(pairs):
        seg = seg_h if hi else seg_l
        a, b = (masked(gp[i], cfg) if first else gp[i]), op[i]
        if np.array_equal(a, b):
            continue
        assert not scores_exact, f"{what}: page pair {i} differs"
        a2, b2 = a.copy(), b.copy()
        a2[seg[4]:seg[5]] = 0
        b2[seg[4]:seg[5]] = 0
        assert np.array_equal(a2, b2), f"{what}: page pair {i} differs outside the score segment"
        sa, sb = a[seg[4]:seg[5]].view(np.float32), b[seg[4]:seg[5]].view(np.float32)
        assert np.all(np.abs(sa - sb) <= SCORE_ATOL + SCORE_RTOL * np.abs(sb)), \
            f"{what}: page pair {i} score sums differ beyond tolerance"
    return pairs


def resync_sampled(g, o, pairs):
    """Oracle page bytes into the device pages of the sampled requests, so
    the next step decides from identical score sums."""
    if not pairs:
        return
    pages = g.pool.pages.view(g.pool.num_pages, -1)
    gid = torch.tensor([p[0] for p in pairs], dtype=torch.int64, device=dev)
    pages[gid] = torch.from_numpy(o.pages[[p[1] for p in pairs]]).to(dev)
    torch.cuda.synchronize()


def sub_prompt(pr, sample, H):
    """Host arrays of the sampled requests' prompt slices."""
    cu = pr["cu_seqlens"].numpy()
    ks, vs, ss = [], [], []
    lens = []
    for r in sample:
        a, b = int(cu[r]), int(cu[r + 1])
        ks.append(pr["k"][a:b].cpu())
        vs.append(pr["v"][a:b].cpu())
        ss.append(pr["scores"][:, a:b].cpu())
        lens.append(b - a)
    cu_s = np.zeros(len(sample) + 1, np.int64)
    cu_s[1:] = np.cumsum(lens)
    return (cu_s, torch.cat(ks).numpy(), torch.cat(vs).numpy(), torch.cat(ss, dim=1).numpy())


def device_prompt(g, pr):
    cu = pr["cu_seqlens"].to(dev)
    tiers, counts = g.classify(cu, pr["scores"])
    g.compact_prompt(cu, pr["k"], pr["v"], pr["scores"], tiers)
    torch.cuda.synchronize()
    assert int(np_(g.pool.status)[0]) == 0
    return np_(counts)


def oracle_prompt(orc, o, cfg, sub):
    cu_s, k, v, sc = sub
    tiers, counts = orc.classify(cfg, cu_s, sc)
    o.compact_prompt(cu_s, k, v, sc, tiers)
    assert int(o.status[0]) == 0
    return counts


def run_sampled(dk, orc, cfg, sample, steps, what, ptr_offset=0, events=None):
    """Full batch on the device, sampled requests on the oracle; `steps`
    decode steps (STEP compaction, attention with the score update).
    events: {step: [requests released and re-admitted before that step]}."""
    from workloads import synth
    B, H, G, d = cfg["batch"], cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    lens = synth.seq_lens(cfg)
    pr = synth.make_prompt(cfg, device=dev, lens=lens)
    P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
    g = dk.DiffKVState(cfg, B, P, max_total_tokens=max(int(lens.sum()), 16000 * 8), device=dev)
    if ptr_offset:
        # start both counters deep into the list: every list index wraps
        off = (ptr_offset // P) * P + (P - 777 % P)
        g.pool.ptr.copy_(torch.tensor([off, off + P], dtype=torch.int64, device=dev))
    _say(f"{what}: B={B} P={P} units={B * H} splits={dk.diffkv_attn_splits(cfg, B)}")
    counts = device_prompt(g, pr)
    sub = sub_prompt(pr, sample, H)
    del pr
    _free_gpu()
    o = orc.State(cfg, len(sample), 64 + 2 * sum(-(-int(n) // 16) for n in np.diff(sub[0])) * H)
    counts_o = oracle_prompt(orc, o, cfg, sub)
    assert np.array_equal(counts[sample], counts_o), f"{what}: tier counts differ"
    pairs = compare_sampled(g, o, orc, cfg, sample, True, f"{what} prompt")
    check_device_pool(g)
    seq = lens.numpy().astype(np.int32)
    for step in range(steps):
        for r in (events or {}).get(step, []):
            # release request r and admit a fresh prompt in its slot
            mask = np.zeros(B, np.uint8)
            mask[r] = 1
            g.release(torch.from_numpy(mask).to(dev))
            newlen = 1000 + (7919 * (r + 1) * (step + 3)) % 15001
            cfg1 = dict(cfg, batch=1)
            pr1 = synth.make_prompt(cfg1, device=dev, salt=50 + step, lens=torch.tensor([newlen]))
            lens_b = torch.zeros(B, dtype=torch.int64)
            lens_b[r] = newlen
            cu_b = torch.zeros(B + 1, dtype=torch.int64)
            cu_b[1:] = torch.cumsum(lens_b, 0)
            tiers, _ = g.classify(cu_b.to(dev), pr1["scores"])
            g.compact_prompt(cu_b.to(dev), pr1["k"], pr1["v"], pr1["scores"], tiers)
            seq[r] = newlen
            if r in sample:
                i = sample.index(r)
                mo = np.zeros(len(sample), np.uint8)
                mo[i] = 1
                o.release(mo)
                lens_o = np.zeros(len(sample), np.int64)
                lens_o[i] = newlen
                cu_o = np.zeros(len(sample) + 1, np.int64)
                cu_o[1:] = np.cumsum(lens_o)
                sc = pr1["scores"].cpu().numpy()
                t_o, _ = orc.classify(cfg, cu_o, sc)
                o.compact_prompt(cu_o, pr1["k"].cpu().numpy(), pr1["v"].cpu().numpy(), sc, t_o)
            del pr1
            torch.cuda.synchronize()
            assert int(np_(g.pool.status)[0]) == 0, f"{what}: re-admission status"
        dec = synth.make_decode(cfg, step, device=dev)
        sq = torch.from_numpy(seq).to(dev)
        g.compact_step(sq, dec["k_new"], dec["v_new"])
        out = g.decode_attn(dec["q"], sq, update_scores=1)
        torch.cuda.synchronize()
        assert int(np_(g.pool.status)[0]) == 0, f"{what}: step {step} status"
        so = seq[sample]
        o.compact_step(so, np_(dec["k_new"])[sample], np_(dec["v_new"])[sample])
        out_o = o.decode_attn(np_(dec["q"])[sample], so, update_scores=True)
        err = assert_attn_close(np_(out)[sample], out_o, f"{what} attn {step}")
        pairs = compare_sampled(g, o, orc, cfg, sample, False, f"{what} step {step}")
        resync_sampled(g, o, pairs)
        _say(f"  step {step}: attention max err {err:.2e}, {len(pairs)} sampled pages equal")
        seq = seq + 1
    check_device_pool(g)
    del g
    _free_gpu()


# --------------------------------------------------------------------------
# tests
# --------------------------------------------------------------------------
def _clone_state(dk, g, cfg, B, P, total):
    """A second device cache with g's tables, tier state and pool bytes."""
    c = dk.DiffKVState(cfg, B, P, max_total_tokens=total, device=dev)
    for name in ("page_table", "tier_state"):
        getattr(c, name).copy_(getattr(g, name))
    for name in ("pages", "free_list", "ptr", "status"):
        getattr(c.pool, name).copy_(getattr(g.pool, name))
    torch.cuda.synchronize()
    return c


def test_llama3_8b_full_batch(dk, orc):
    """Whole Llama3-8B-shaped batch on both sides: bit-exact state and pages,
    attention and scores within tolerance, for two decode steps through the
    separate calls and one through diffkv_decode_step (the fused kernel, plan
    kernel first).  Then the launch configuration the benchmark times --
    chained decode steps, planned by the previous step's attention -- for
    three steps against a copy of the cache stepping through the plan kernel:
    outputs and caches byte-identical."""
    from workloads import synth
    from tests.test_gpu_parity import Pair
    cfg = synth.config("llama3_8b")
    B = cfg["batch"]
    lens = synth.seq_lens(cfg)
    pr = synth.make_prompt(cfg, device=dev, lens=lens)
    P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
    assert dk.diffkv_attn_splits(cfg, B) == 1
    p = Pair(dk, orc, cfg, B, P, int(lens.sum()))
    _say(f"llama3_8b full: P={P}")
    cu = pr["cu_seqlens"].numpy()
    p.prompt(cu, np_(pr["k"]), np_(pr["v"]), np_(pr["scores"]))
    del pr
    _free_gpu()
    check_device_pool(p.g)
    seq = lens.numpy().astype(np.int32)
    for step in range(2):
        dec = synth.make_decode(cfg, step)
        p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
        err = p.attend(dec["q"].numpy(), seq, True, f"attn {step}")
        _say(f"  step {step}: attention max err {err:.2e}")
        seq = seq + 1
    dec = synth.make_decode(cfg, 2)
    err = p.decode_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy(), True,
                        "fused decode step 2")
    _say(f"  fused decode step 2: attention max err {err:.2e}")
    seq = seq + 1
    check_device_pool(p.g)
    a_ = p.g
    del p.o
    b_ = _clone_state(dk, a_, cfg, B, P, int(lens.sum()))
    sd = torch.from_numpy(seq).to(dev)
    for step in range(3, 6):
        dec = synth.make_decode(cfg, step, device=dev)
        oa = a_.decode_step(dec["q"], sd, dec["k_new"], dec["v_new"], update_scores=1)
        ob = b_.decode_step(dec["q"], sd, dec["k_new"], dec["v_new"], update_scores=1, chain=0)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"chained step {step}: outputs differ"
        for name in ("page_table", "tier_state"):
            assert torch.equal(getattr(a_, name), getattr(b_, name)), f"chained step {step}: {name} differs"
        assert torch.equal(a_.pool.free_list, b_.pool.free_list) and torch.equal(a_.pool.ptr, b_.pool.ptr)
        assert torch.equal(a_.pool.pages, b_.pool.pages), f"chained step {step}: pages differ"
        _say(f"  chained step {step}: identical (chain {a_.chain})")
        sd = sd + 1
    assert a_.chain == 3 and int(a_.pool.status.item()) == 0
    check_device_pool(a_)
    del p, a_, b_
    _free_gpu()


def test_long_context_sampled(dk, orc):
    from workloads import synth
    cfg = synth.config("long")
    assert dk.diffkv_attn_splits(cfg, cfg["batch"]) > 1
    run_sampled(dk, orc, cfg, [1, 6], 2, "long")


def test_churn_sampled_with_release_and_wrap(dk, orc):
    from workloads import synth
    cfg = synth.config("churn")
    run_sampled(dk, orc, cfg, [3, 40, 77, 127], 4, "churn", ptr_offset=10**9,
                events={1: [40, 90], 2: [3]})


@pytest.mark.parametrize("name", ["stress_gqa7", "stress_gqa8"])
def test_stress_sampled(dk, orc, name):
    from workloads import synth
    cfg = synth.config(name)
    run_sampled(dk, orc, cfg, [5, 33], 2, name)
