"""Chained decode steps against the oracle, step by step.

A chained diffkv_decode_step (the launch configuration bench.py times) runs
no plan kernel: the previous step's attention planned it from the score sums
it had just written.  These tests compare every such step with the oracle's
STEP followed by attention with the score update (DiffKV notes, "KV
compression policy": generation phase and algorithm flow; "Memory
management": generation workflow; "Implementation": compaction before the
attention kernel):

* state bit-exact after every step: page tables, tier state, free list, both
  pointers, status, and every live page byte outside the score segment;
* attention outputs within 2e-3 + 1e-3 |ref|, score sums within
  1e-5 + 1e-4 |ref|;
* then the device's score sums are copied into the oracle's pages, so both
  sides decide the next step from the same sums while the device's chain
  stays live (fp32 sums agree to a tolerance, not bit for bit).

The oracle records which case of the generation-phase policy each unit took,
and the tests assert that every case occurred.
"""
import numpy as np
import pytest
import torch

from tests.invariants import check_pool_invariants
from tests.parity import (assert_attn_close, assert_state_equal, compare_pages_scores_tol, np_,
                          sync_scores_to_oracle)

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


BR_NAMES = ["inactive", "no t_c", "hi/keep", "hi/demote", "hi/prune", "lo/keep", "lo/prune", "prune"]


def _count(br, acc):
    for x in br.ravel():
        acc["case"][int(x) & 15] += 1
        acc["page"][(int(x) >> 4) & 3] += 1


def _report(acc):
    cases = {BR_NAMES[i]: int(c) for i, c in enumerate(acc["case"]) if c}
    return f"cases {cases}, new pages hi {int(acc['page'][2])} lo {int(acc['page'][1])}"


def run_chained(dk, orc, cfg, lens, steps, q_scale, what):
    """Prompt compaction on both sides, then `steps` chained decode steps on
    the device, each compared with the oracle.  Returns the branch counts."""
    from workloads import synth
    B = int(lens.numel())
    H = cfg["num_kv_heads"]
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    if "pool_factor" in cfg:
        P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
    else:
        P = int(sum(-(-(int(n) + steps) // 16) + 2 for n in lens) * H * 1.3) + 16
    assert dk.diffkv_attn_splits(cfg, B) == 1
    g = dk.DiffKVState(cfg, B, P, max_total_tokens=int(cu[-1]), device=dev)
    o = orc.State(cfg, B, P)
    sc = pr["scores"].numpy()
    tiers_o, _ = orc.classify(cfg, cu, sc)
    o.compact_prompt(cu, pr["k"].numpy(), pr["v"].numpy(), sc, tiers_o)
    cu_d = torch.from_numpy(cu).to(dev)
    sc_d = torch.from_numpy(sc).to(dev)
    tiers, _ = g.classify(cu_d, sc_d)
    g.compact_prompt(cu_d, pr["k"].to(dev), pr["v"].to(dev), sc_d, tiers)
    torch.cuda.synchronize()
    assert_state_equal(g, o, what=f"{what} prompt")
    acc = {"case": np.zeros(8, np.int64), "page": np.zeros(4, np.int64)}
    seq = lens.numpy().astype(np.int32)
    worst_attn = worst_score = 0.0
    for step in range(steps):
        dec = synth.make_decode(cfg, step, q_scale=q_scale)
        kn, vn, q = dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy()
        br = o.compact_step(seq, kn, vn, branches=True)
        out_o = o.decode_attn(q, seq, update_scores=True)
        chain_before = g.chain
        out_g = g.decode_step(torch.from_numpy(q).to(dev), torch.from_numpy(seq).to(dev),
                              torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev), update_scores=1)
        torch.cuda.synchronize()
        assert chain_before == step, f"{what} step {step}: chain {chain_before}"
        _count(br, acc)
        assert_state_equal(g, o, pages=False, what=f"{what} step {step}")
        worst_attn = max(worst_attn, assert_attn_close(out_g, out_o, f"{what} step {step}"))
        worst_score = max(worst_score, compare_pages_scores_tol(g, o, f"{what} step {step}"))
        sync_scores_to_oracle(g, o)
        seq = seq + 1
    assert g.chain == steps
    check_pool_invariants(orc, o)
    _say(f"{what}: {steps} chained steps, attention max err {worst_attn:.2e}, "
         f"worst score ratio {worst_score:.2f}; {_report(acc)}")
    del g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return acc


CHAIN_CASES = [(128, 4, 1), (64, 5, 1), (128, 7, 0), (128, 8, 1), (64, 16, 1)]
_BRANCHES = {}


@pytest.mark.parametrize("d,G,lo", CHAIN_CASES)
def test_chained_decode_steps_vs_oracle(dk, orc, d, G, lo):
    """64 chained decode steps on a ragged batch (prompts of 383, 37, 20, 127
    and 14 tokens: tails inside pages, prompts shorter than the window).
    Queries are drawn 3x sharper than N(0, 1) and the window is 8 tokens, so
    that tokens lose importance within the run and every policy case occurs."""
    from workloads import synth
    cfg = synth.config("llama3_8b", head_dim=d, gqa_group=G, lo_enabled=lo, num_kv_heads=3, batch=5,
                       max_seq_len=480, window=8)
    cfg.pop("pool_factor")
    lens = torch.tensor([383, 37, 20, 127, 14], dtype=torch.int64)
    acc = run_chained(dk, orc, cfg, lens, 64, 3.0, f"chained d={d} G={G} lo={lo}")
    _BRANCHES[(d, G, lo)] = acc
    c = acc["case"]
    for k in (2, 7):                      # hi/keep, prune
        assert c[k] > 0, f"case {BR_NAMES[k]} never occurred: {_report(acc)}"
    assert acc["page"][2] > 0, f"no high page growth: {_report(acc)}"
    if lo:
        for k in (3, 5, 6):               # hi/demote, lo/keep, lo/prune
            assert c[k] > 0, f"case {BR_NAMES[k]} never occurred: {_report(acc)}"
    else:
        assert c[4] > 0, f"case hi/prune never occurred: {_report(acc)}"
        assert c[3] == c[5] == c[6] == 0 and acc["page"][1] == 0


def test_chained_branch_union():
    """Over the five configurations: every case of the generation-phase
    policy, and page growth in both tiers."""
    if len(_BRANCHES) < len(CHAIN_CASES):
        pytest.skip("needs every configuration of test_chained_decode_steps_vs_oracle in this session")
    case = sum(a["case"] for a in _BRANCHES.values())
    page = sum(a["page"] for a in _BRANCHES.values())
    _say("union:", {BR_NAMES[i]: int(x) for i, x in enumerate(case)}, "pages hi", int(page[2]), "lo", int(page[1]))
    assert all(case[k] > 0 for k in range(2, 8))
    assert page[1] > 0 and page[2] > 0


def test_llama3_8b_chained_vs_oracle(dk, orc):
    """The benchmark's workload (Llama3-8B-shaped layer: B32, 4096 tokens,
    8 KV heads, GQA 4, d = 128), whole batch on both sides, 16 chained decode
    steps each compared with the oracle."""
    from workloads import synth
    cfg = synth.config("llama3_8b")
    lens = synth.seq_lens(cfg)
    run_chained(dk, orc, cfg, lens, 16, 1.0, "llama3_8b chained")


def test_score_update_max_over_group_on_device(dk, orc):
    """The worked case of the oracle's score-update pin on the device: five
    high tokens with constant keys (+1 for token 2, -1 otherwise), two q
    heads, one 3 in every dim (all its weight on token 2), one zero (weights
    exactly 1/5).  The group's weight is the max over its heads: token 2
    gains 1.0, the others 0.2, the query's own token (position 4) nothing."""
    for d in (64, 128):
        n, G = 5, 2
        cfg = dict(head_dim=d, num_kv_heads=1, gqa_group=G, max_seq_len=64, window=0,
                   alpha_h=1.0, alpha_l=0.2)
        k = np.where(np.arange(n)[:, None] == 2, 1.0, -1.0) * np.ones((n, 1, d))
        rng = np.random.default_rng(12)
        v = rng.standard_normal((n, 1, d))
        kb = k.astype(np.float16).view(np.int16)
        vb = v.astype(np.float16).view(np.int16)
        g = dk.DiffKVState(cfg, 1, 8, max_total_tokens=n, device=dev)
        cu = torch.tensor([0, n], dtype=torch.int64, device=dev)
        sc = torch.zeros(1, n, dtype=torch.float32, device=dev)
        tiers = torch.full((1, n), 2, dtype=torch.uint8, device=dev)
        g.compact_prompt(cu, torch.from_numpy(kb).to(dev), torch.from_numpy(vb).to(dev), sc, tiers)
        q = np.zeros((1, G, d), np.float16)
        q[0, 0] = 3.0
        g.decode_attn(torch.from_numpy(q.view(np.int16)).to(dev), torch.tensor([4], dtype=torch.int32, device=dev),
                      update_scores=1)
        torch.cuda.synchronize()
        from oracle import tier_layout, HI
        _, seg = tier_layout(cfg, HI)
        page = np_(g.pool.pages.view(g.pool.num_pages, -1))[int(np_(g.page_table)[0, 0, 0])]
        pos = page[seg[5]:seg[5] + 4 * n].view(np.int32)
        got = page[seg[4]:seg[4] + 4 * n].view(np.float32)
        by_pos = dict(zip(pos.tolist(), got.tolist()))
        expect = {0: 0.2, 1: 0.2, 2: 1.0, 3: 0.2, 4: 0.0}
        for p_, e in expect.items():
            assert abs(by_pos[p_] - e) <= 1e-5 + 1e-4 * e, f"d={d}: position {p_} score {by_pos[p_]} vs {e}"
        assert int(np_(g.pool.status)[0]) == 0


@pytest.mark.parametrize("bad_id", [-1, "P"])
def test_release_rejects_page_ids_outside_the_pool(dk, orc, bad_id):
    """A released unit whose table row holds a page id outside the pool:
    BAD_STATE on both sides and nothing committed (tables, tier state, free
    list and pointers unchanged)."""
    from workloads import synth
    cfg = synth.config("llama3_8b", num_kv_heads=3, batch=4, max_seq_len=1200, window=64)
    cfg.pop("pool_factor")
    lens = torch.tensor([700, 37, 300, 1000], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) + 2 for n in lens) * 3 * 1.2) + 8
    from tests.test_gpu_parity import Pair
    p = Pair(dk, orc, cfg, 4, P, int(cu[-1]))
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    L = p.o.page_table.shape[-1]
    idv = -1 if bad_id == -1 else P
    # request 2, head 1: its innermost low page's entry (a used entry)
    pl = int(p.o.tier_state[2, 1, 3])
    assert pl > 0
    p.o.page_table[2, 1, L - pl] = idv
    p.g.page_table[2, 1, L - pl] = idv
    before = p.o.copy()
    p.release(np.array([1, 0, 1, 1], np.uint8), what="release with a bad id")
    assert int(p.o.status[0]) == orc.ST_BAD_STATE
    assert np.array_equal(p.o.page_table, before.page_table)
    assert np.array_equal(p.o.free_list, before.free_list) and np.array_equal(p.o.ptr, before.ptr)


def test_split_chain_reuses_dispatch_order(dk):
    """Several splits per unit and more (unit, split) pairs than compute
    units: a chained diffkv_decode_step keeps the dispatch order (units by
    page count) the chain's first call left in the workspace and recomputes
    it every 16 calls.  The order changes timing only, so 20 chained steps
    and the same 20 steps each with chain = 0 (order recomputed every time)
    must leave byte-identical outputs, tables, tier state, pool and pages."""
    from workloads import synth
    cfg = synth.config("llama3_8b", num_kv_heads=8, batch=3, max_seq_len=4200, window=64)
    cfg.pop("pool_factor", None)
    B, H = 3, 8
    S = dk.diffkv_attn_splits(cfg, B)
    assert S > 1 and B * H * S > 256, (S, B * H)
    lens = torch.tensor([3500, 1200, 2700], dtype=torch.int64)
    pr = synth.make_prompt(cfg, device=dev, lens=lens)
    P = int(sum(-(-int(n) // 16) for n in lens) * H * 1.2) + 64
    cu = pr["cu_seqlens"].to(dev)
    a = dk.DiffKVState(cfg, B, P, max_total_tokens=int(lens.sum()), device=dev)
    t, _ = a.classify(cu, pr["scores"])
    a.compact_prompt(cu, pr["k"], pr["v"], pr["scores"], t)
    # the second cache: a byte copy of the first (pages never written included)
    b = dk.DiffKVState(cfg, B, P, max_total_tokens=int(lens.sum()), device=dev)
    for name in ("page_table", "tier_state"):
        getattr(b, name).copy_(getattr(a, name))
    for name in ("pages", "free_list", "ptr", "status"):
        getattr(b.pool, name).copy_(getattr(a.pool, name))
    torch.cuda.synchronize()
    seq = lens.to(torch.int32).to(dev)
    for step in range(20):
        dec = synth.make_decode(cfg, step, device=dev)
        oa = a.decode_step(dec["q"], seq, dec["k_new"], dec["v_new"], update_scores=1)
        ob = b.decode_step(dec["q"], seq, dec["k_new"], dec["v_new"], update_scores=1, chain=0)
        torch.cuda.synchronize()
        what = f"split chain step {step} (chain {a.chain})"
        assert torch.equal(oa, ob), f"{what}: outputs differ"
        for name in ("page_table", "tier_state"):
            assert torch.equal(getattr(a, name), getattr(b, name)), f"{what}: {name} differs"
        assert torch.equal(a.pool.free_list, b.pool.free_list) and torch.equal(a.pool.ptr, b.pool.ptr), what
        assert torch.equal(a.pool.pages, b.pool.pages), f"{what}: pages differ"
        seq = seq + 1
    assert a.chain == 20 and int(a.pool.status.item()) == 0 and int(b.pool.status.item()) == 0
    _say(f"split chain: S={S}, 20 chained steps identical to unchained ones")
