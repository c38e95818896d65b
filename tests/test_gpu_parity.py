"""GPU parity of the C-ABI library against the oracle (small and medium sizes
that span several pages, splits and ragged tails).

Bit-exact: tiers, tier counts, page tables, tier state, free list, both
pointers, status, and every byte of every live page after compaction.
Tolerance: attention outputs |gpu - ref| <= 2e-3 + 1e-3 |ref|; score sums
after the update 1e-5 + 1e-4 |ref| (then re-synced to the oracle's bytes).
"""
import numpy as np
import pytest
import torch

from tests.invariants import check_pool_invariants
from tests.parity import (assert_attn_close, assert_scores_close, assert_state_equal, np_,
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


def _scores_for(cfg, pr, orc):
    from workloads import synth
    if cfg["score"] == "probe":
        return orc.importance_from_queries(cfg, pr["cu_seqlens"].numpy(), pr["k"].numpy(),
                                           synth.probe_queries(cfg).numpy())
    return pr["scores"].numpy()


class Pair:
    """The same cache on the device (library) and on the host (oracle)."""

    def __init__(self, dk, orc, cfg, batch, num_pages, max_total):
        self.cfg, self.batch = cfg, batch
        self.g = dk.DiffKVState(cfg, batch, num_pages, max_total_tokens=max_total, device=dev)
        self.o = orc.State(cfg, batch, num_pages)
        self.orc = orc

    def prompt(self, cu, k, v, scores, check=True, what="prompt"):
        tiers_o, counts_o = self.orc.classify(self.cfg, cu, scores)
        sc = torch.from_numpy(np.ascontiguousarray(scores)).to(dev)
        cu_d = torch.from_numpy(np.ascontiguousarray(cu, dtype=np.int64)).to(dev)
        tiers, counts = self.g.classify(cu_d, sc)
        assert np.array_equal(np_(tiers), tiers_o), f"{what}: tiers differ"
        assert np.array_equal(np_(counts), counts_o), f"{what}: counts differ"
        self.o.compact_prompt(cu, k, v, scores, tiers_o)
        self.g.compact_prompt(cu_d, torch.from_numpy(np.ascontiguousarray(k)).to(dev),
                              torch.from_numpy(np.ascontiguousarray(v)).to(dev), sc, tiers)
        torch.cuda.synchronize()
        if check:
            assert_state_equal(self.g, self.o, what=what)

    def step(self, seq, kn, vn, what="step"):
        self.o.compact_step(seq, kn, vn)
        self.g.compact_step(torch.from_numpy(seq).to(dev), torch.from_numpy(kn).to(dev),
                            torch.from_numpy(vn).to(dev))
        torch.cuda.synchronize()
        assert_state_equal(self.g, self.o, what=what)

    def attend(self, q, seq, update, what="attn"):
        out_o = self.o.decode_attn(q, seq, update_scores=update)
        out_g = self.g.decode_attn(torch.from_numpy(q).to(dev), torch.from_numpy(seq).to(dev),
                                   update_scores=update)
        torch.cuda.synchronize()
        err = assert_attn_close(out_g, out_o, what)
        if update:
            assert_scores_close(self.g, self.o, what)
            resync_scores(self.g, self.o)
        return err

    def decode_step(self, seq, kn, vn, q, update, what="decode step"):
        """diffkv_decode_step against the oracle's STEP followed by attention."""
        self.o.compact_step(seq, kn, vn)
        out_o = self.o.decode_attn(q, seq, update_scores=update)
        out_g = self.g.decode_step(torch.from_numpy(q).to(dev), torch.from_numpy(seq).to(dev),
                                   torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev),
                                   update_scores=1 if update else 0)
        torch.cuda.synchronize()
        assert_state_equal(self.g, self.o, pages=not update, what=what)
        err = assert_attn_close(out_g, out_o, what)
        if update:
            assert_scores_close(self.g, self.o, what)
            resync_scores(self.g, self.o)
        return err

    def release(self, mask, what="release"):
        self.o.release(mask)
        self.g.release(torch.from_numpy(np.asarray(mask, np.uint8)).to(dev))
        torch.cuda.synchronize()
        assert_state_equal(self.g, self.o, pages=False, what=what)


def test_smoke_entry():
    import __graft_entry__
    __graft_entry__.smoke()


@pytest.mark.parametrize("window", [64, 0])
def test_tiny_prompt_and_attention(dk, orc, window):
    from workloads import synth
    cfg = synth.config("tiny", window=window)
    pr = synth.make_prompt(cfg)
    sc = _scores_for(cfg, pr, orc)
    p = Pair(dk, orc, cfg, 1, 64, int(pr["cu_seqlens"][-1]))
    _say("tiny prompt, W =", window)
    p.prompt(pr["cu_seqlens"].numpy(), pr["k"].numpy(), pr["v"].numpy(), sc)
    check_pool_invariants(orc, p.o)
    dec = synth.make_decode(cfg, 0)
    seq = pr["lens"].numpy().astype(np.int32)
    err = p.attend(dec["q"].numpy(), seq - 1, False, "tiny attn")
    _say("tiny attention max err", err)


def _edge_rows(rng, n, d, tiers, kv):
    """fp16 rows that sit on the codec's edges, cycling over the row types:
    random; constant (zero scale); a range below fp16 resolution (subnormal
    or zero scale); subnormal values; the full +-65504 range; a large offset
    with a small range; and rows whose quotients (x - z) / s are exact
    half-integers for the code width of the token's tier (ties to even).
    `kv` = 0 for K, 1 for V; tiers: 2 high, 1 low, 0 pruned."""
    out = np.zeros((n, d), np.float32)
    for t in range(n):
        kind = t % 7
        if kind == 0:
            r = rng.standard_normal(d)
        elif kind == 1:
            r = np.full(d, rng.standard_normal() * 3)
        elif kind == 2:
            r = 1.0 + rng.standard_normal(d) * 1e-5
        elif kind == 3:
            r = rng.standard_normal(d) * 1e-6
        elif kind == 4:
            r = rng.standard_normal(d) * 1000
            r[rng.integers(0, d)] = 65504.0
            r[rng.integers(0, d)] = -65504.0
        elif kind == 5:
            r = 1000.0 + rng.standard_normal(d) * 0.5
        else:
            bits = {(2, 0): 8, (2, 1): 4, (1, 0): 4, (1, 1): 2}.get((int(tiers[t]), kv), 8)
            q = (1 << bits) - 1
            r = (rng.integers(0, q, d) + 0.5) * 0.25   # exact half-integer quotients
            i0, i1 = rng.choice(d, 2, replace=False)
            r[i0], r[i1] = 0.0, q * 0.25               # min 0, max q s: s = 0.25 exactly
        out[t] = r
    return out.astype(np.float16)


@pytest.mark.parametrize("d", [128, 64])
def test_prompt_codec_edge_rows(dk, orc, d):
    """Prompt compaction of rows on the codec's edges (constant, sub-resolution
    and subnormal ranges, +-65504, large offsets, exact half-integer
    quotients) is byte-identical to the oracle: codes, fp16 scale/zero,
    scores, positions and every page."""
    from workloads import synth
    cfg = synth.config("llama3_8b", head_dim=d, num_kv_heads=2, batch=2, window=0, max_seq_len=512)
    lens = np.array([200, 77])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total, H = int(cu[-1]), 2
    rng = np.random.default_rng(20261202)
    # tiers by score (window 0): t % 3 -> high, low, pruned
    scores = np.zeros((H, total), np.float32)
    tiers = np.zeros((H, total), np.int64)
    for b in range(2):
        N = int(lens[b])
        for h in range(H):
            for t in range(N):
                tiers[h, cu[b] + t] = (2, 1, 0)[(t + h) % 3]
                scores[h, cu[b] + t] = {2: 2.0, 1: 0.5, 0: 0.05}[tiers[h, cu[b] + t]] / N
    k = np.zeros((total, H, d), np.float16)
    v = np.zeros((total, H, d), np.float16)
    for h in range(H):
        k[:, h] = _edge_rows(rng, total, d, tiers[h], 0)
        v[:, h] = _edge_rows(rng, total, d, tiers[h], 1)
    p = Pair(dk, orc, cfg, 2, 64, total)
    _say(f"codec edge rows d={d}")
    p.prompt(cu, k.view(np.int16), v.view(np.int16), scores, what=f"edge rows d={d}")
    check_pool_invariants(orc, p.o)


def _medium_cfg(name, **over):
    from workloads import synth
    c = synth.config(name, **over)
    return c


@pytest.mark.parametrize("d,G,lo", [(128, 4, 1), (64, 5, 1), (128, 7, 0), (128, 8, 1), (64, 16, 1)])
def test_ragged_prompt_step_attention(dk, orc, d, G, lo):
    """Ragged batch (tails inside pages, a prompt shorter than the window),
    prompt compaction, 6 steps with score updates, release of half the batch,
    re-admission into the freed slots."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", head_dim=d, gqa_group=G, lo_enabled=lo, num_kv_heads=3,
                      batch=5, max_seq_len=3000, window=64)
    lens = torch.tensor([1500, 37, 700, 1201, 64], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    sc = pr["scores"].numpy()
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 3 * 1.1) + 8
    p = Pair(dk, orc, cfg, 5, P, int(cu[-1]))
    _say(f"ragged d={d} G={G} lo={lo}: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), sc)
    check_pool_invariants(orc, p.o)
    seq = lens.numpy().astype(np.int32)
    for step in range(6):
        dec = synth.make_decode(cfg, step)
        _say("  step", step)
        p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
        p.attend(dec["q"].numpy(), seq, True, f"attn {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)
    mask = np.array([1, 0, 1, 0, 1], np.uint8)
    p.release(mask)
    check_pool_invariants(orc, p.o)
    lens2 = torch.tensor([900, 0, 65, 0, 333], dtype=torch.int64)
    pr2 = synth.make_prompt(cfg, lens=lens2, salt=7)
    _say("  re-admit")
    p.prompt(pr2["cu_seqlens"].numpy(), pr2["k"].numpy(), pr2["v"].numpy(), pr2["scores"].numpy(),
             what="re-admit")
    check_pool_invariants(orc, p.o)
    seq = np.where(mask == 1, lens2.numpy(), seq).astype(np.int32)
    dec = synth.make_decode(cfg, 99)
    p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), "step after re-admit")
    p.attend(dec["q"].numpy(), seq, True, "attn after re-admit")


@pytest.mark.parametrize("d,G,lo", [(128, 4, 1), (64, 5, 1), (128, 7, 0), (128, 8, 1), (64, 16, 1)])
def test_decode_step_fused_variants(dk, orc, d, G, lo):
    """diffkv_decode_step through the fused kernel (short rows: one split per
    unit) for both head sizes, both weight-column layouts (2G <= 16 or not)
    and the low tier off; ragged lengths with tails inside pages, steps that
    cross page boundaries, then release and re-admission."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", head_dim=d, gqa_group=G, lo_enabled=lo, num_kv_heads=3,
                      batch=5, max_seq_len=420, window=64)
    assert dk.diffkv_attn_splits(cfg, 5) == 1
    lens = torch.tensor([383, 37, 200, 127, 64], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) + 2 for n in lens) * 3 * 1.2) + 8
    p = Pair(dk, orc, cfg, 5, P, int(cu[-1]))
    _say(f"fused decode step d={d} G={G} lo={lo}: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    for step in range(8):
        dec = synth.make_decode(cfg, step)
        _say("  decode step", step)
        p.decode_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy(), True,
                      f"decode step {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)
    mask = np.array([1, 0, 0, 1, 0], np.uint8)
    p.release(mask)
    lens2 = torch.tensor([95, 0, 0, 300, 0], dtype=torch.int64)
    pr2 = synth.make_prompt(cfg, lens=lens2, salt=5)
    p.prompt(pr2["cu_seqlens"].numpy(), pr2["k"].numpy(), pr2["v"].numpy(), pr2["scores"].numpy(),
             what="re-admit")
    seq = np.where(mask == 1, lens2.numpy(), seq).astype(np.int32)
    for step in range(3):
        dec = synth.make_decode(cfg, 50 + step)
        p.decode_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy(), step != 1,
                      f"decode step after re-admit {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)


def test_fig6_scaled_on_gpu(dk, orc):
    """The Fig 6 worked example at 16/32-token pages: pages 5-8 to head A,
    9-12 to head B, pointer to 13, pages 6, 7, 11 reclaimed."""
    cfg = dict(head_dim=128, num_kv_heads=2, gqa_group=1, max_seq_len=64, window=0,
               alpha_h=1.0, alpha_l=0.2)
    N = 64
    tiers = np.zeros((2, N), np.uint8)
    tiers[0, :16] = 2
    tiers[0, 16:40] = 1
    tiers[1, 0:17] = 2
    tiers[1, 30:50] = 1
    rng = np.random.default_rng(3)
    k = rng.standard_normal((N, 2, 128)).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((N, 2, 128)).astype(np.float16).view(np.uint16)
    scores = rng.random((2, N)).astype(np.float32) / N
    g = dk.DiffKVState(cfg, 1, 16, max_total_tokens=N, device=dev)
    g.pool.ptr[0] = 5                                  # pages 0-4 in use
    g.compact_prompt(torch.tensor([0, N], device=dev), torch.from_numpy(k).to(dev),
                     torch.from_numpy(v).to(dev), torch.from_numpy(scores).to(dev),
                     torch.from_numpy(tiers).to(dev))
    torch.cuda.synchronize()
    pt = np_(g.page_table)
    assert pt[0, 0].tolist() == [5, -1, -1, -1, 8]
    assert pt[0, 1].tolist() == [9, 10, -1, -1, 12]
    assert np_(g.pool.ptr).tolist() == [13, 19]
    assert np_(g.pool.free_list)[:3].tolist() == [6, 7, 11]


def test_exhaustion_and_overflow_commit_nothing(dk, orc):
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", num_kv_heads=2, batch=2, max_seq_len=600)
    lens = torch.tensor([500, 300], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    need = 2 * (-(-500 // 16) - 0) + 2 * (-(-300 // 16))
    p = Pair(dk, orc, cfg, 2, need - 1, int(cu[-1]))
    before = np_(p.g.page_table).copy()
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy(), what="exhausted")
    assert int(p.o.status[0]) == orc.ST_POOL_EXHAUSTED
    assert np.array_equal(np_(p.g.page_table), before)
    # table overflow: a prompt longer than max_seq_len
    cfg2 = dict(cfg, max_seq_len=400)
    p2 = Pair(dk, orc, cfg2, 2, 4 * need, int(cu[-1]))
    p2.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy(), what="overflow")
    assert int(p2.o.status[0]) & orc.ST_TABLE_OVERFLOW


def test_step_exhaustion(dk, orc):
    cfg = dict(head_dim=64, num_kv_heads=1, gqa_group=2, max_seq_len=100, window=64,
               alpha_h=1.0, alpha_l=0.2)
    rng = np.random.default_rng(5)
    N = 32
    k = rng.standard_normal((N, 1, 64)).astype(np.float16).view(np.uint16)
    sc = np.zeros((1, N), np.float32)
    p = Pair(dk, orc, cfg, 1, 2, N)
    p.prompt(np.array([0, N]), k, k, sc)
    kn = k[:1].reshape(1, 1, 64).copy()
    p.step(np.array([N], np.int32), kn, kn, "step exhausted")
    assert int(p.o.status[0]) == orc.ST_POOL_EXHAUSTED


@pytest.mark.parametrize("mode", [1, 2])
def test_single_split_fused_scores(dk, orc, mode):
    """256 units -> one workgroup per unit: attention and score update in one
    kernel (mode 1), or attention keeping logits + diffkv_update_scores (2)."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", batch=32, max_seq_len=1200)
    assert dk.diffkv_attn_splits(cfg, 32) == 1
    g = torch.Generator().manual_seed(11)
    lens = torch.randint(40, 900, (32,), generator=g, dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 8 * 1.1) + 8
    p = Pair(dk, orc, cfg, 32, P, int(cu[-1]))
    _say("single split: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    for step in range(3):
        dec = synth.make_decode(cfg, step)
        p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
        if mode == 1:
            p.attend(dec["q"].numpy(), seq, True, f"attn {step}")
        else:
            out_o = p.o.decode_attn(dec["q"].numpy(), seq, update_scores=True)
            sq = torch.from_numpy(seq).to(dev)
            out_g = p.g.decode_attn(torch.from_numpy(dec["q"].numpy()).to(dev), sq, update_scores=2)
            p.g.update_scores(sq)
            torch.cuda.synchronize()
            assert_attn_close(out_g, out_o, f"attn {step}")
            assert_scores_close(p.g, p.o, f"scores {step}")
            resync_scores(p.g, p.o)
        seq = seq + 1


def test_many_units_coordination_kernel(dk, orc):
    """More units than the commit kernels' own prefix sum covers (2048): the
    step takes the single-block coordination path; one split per unit."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", head_dim=64, num_kv_heads=8, gqa_group=2, batch=264, max_seq_len=400)
    B = 264
    assert B * 8 > 2048 and dk.diffkv_attn_splits(cfg, B) == 1
    g = torch.Generator().manual_seed(21)
    # lengths just below page boundaries so the steps allocate pages
    lens = (torch.randint(5, 12, (B,), generator=g) * 16 - torch.randint(0, 3, (B,), generator=g)).to(torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 8 * 1.2) + 64
    p = Pair(dk, orc, cfg, B, P, int(cu[-1]))
    _say("many units: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    for step in range(4):
        dec = synth.make_decode(cfg, step)
        _say("  step", step)
        if step % 2:  # the decode-step entry: commit inside the attention workgroups
            p.decode_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy(), True,
                          f"decode step {step}")
        else:
            p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
            p.attend(dec["q"].numpy(), seq, True, f"attn {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)


def test_fused_scores_large_units(dk, orc):
    """One split per unit, with units too large to keep their logits in LDS
    (the fused score update then goes through the workspace) next to small
    ones that fit."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", head_dim=64, batch=32, max_seq_len=6400)
    assert dk.diffkv_attn_splits(cfg, 32) == 1
    g = torch.Generator().manual_seed(31)
    lens = torch.where(torch.arange(32) % 2 == 0, torch.randint(5500, 6200, (32,), generator=g),
                       torch.randint(100, 600, (32,), generator=g)).to(torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 8 * 1.05) + 64
    p = Pair(dk, orc, cfg, 32, P, int(cu[-1]))
    _say("large units: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    ts = np_(p.g.tier_state).reshape(-1, 4)
    pages = ts[:, 2] + ts[:, 3]
    G = cfg["gqa_group"]
    assert (pages * 32 * (G + 2) + pages > 16384).any() and (pages * 32 * (G + 2) + pages <= 16384).any()
    seq = lens.numpy().astype(np.int32)
    for step in range(3):
        dec = synth.make_decode(cfg, step)
        if step == 2:  # the decode-step entry (commit inside the attention workgroups)
            p.decode_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy(), True,
                          f"decode step {step}")
        else:
            p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
            p.attend(dec["q"].numpy(), seq, True, f"attn {step}")
        seq = seq + 1


@pytest.mark.parametrize("batch,H,update", [(32, 8, True), (32, 8, False), (64, 8, True), (3, 4, True)])
def test_decode_step_entry(dk, orc, batch, H, update):
    """diffkv_decode_step (STEP then attention in one call): the fused kernel
    when every unit is one split (32 x 8 units: one wave takes the verdict;
    64 x 8: every thread takes part), the separate kernels when not (3 x 4
    units); lengths put steps on page boundaries."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", num_kv_heads=H, batch=batch, max_seq_len=1300)
    assert (dk.diffkv_attn_splits(cfg, batch) == 1) == (batch * H >= 256)
    g = torch.Generator().manual_seed(41)
    lens = (torch.randint(4, 70, (batch,), generator=g) * 16 - torch.randint(0, 2, (batch,), generator=g))
    lens = lens.to(torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * H * 1.1) + 64
    p = Pair(dk, orc, cfg, batch, P, int(cu[-1]))
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    for step in range(4):
        dec = synth.make_decode(cfg, step)
        _say("  decode step", step)
        p.decode_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy(), update,
                      f"decode step {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)


def test_split_units_in_dispatch_order(dk, orc):
    """Several splits per unit with more workgroups than compute units: the
    units are dispatched longest first (and their splits side by side);
    ragged lengths, attention with the score update and decode steps, every
    unit against the oracle."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", num_kv_heads=4, batch=12, max_seq_len=1800)
    S = dk.diffkv_attn_splits(cfg, 12)
    U = 12 * 4
    # more workgroups than this device's compute units: the ordering kernel runs
    assert S > 1 and U * S > torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator().manual_seed(43)
    lens = torch.randint(100, 1700, (12,), generator=g).to(torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 4 * 1.1) + 64
    p = Pair(dk, orc, cfg, 12, P, int(cu[-1]))
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    for step in range(3):
        dec = synth.make_decode(cfg, step)
        _say("  split units, step", step)
        if step == 1:
            p.decode_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy(), True,
                          f"decode step {step}")
        else:
            p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
            p.g.ws_attn.fill_(0xFF)  # no permutation of 0..U-1 left from earlier calls
            p.attend(dec["q"].numpy(), seq, True, f"attn {step}")
            # the dispatch order the attention used: a permutation of the
            # units, longest (most pages) first, somewhere in its workspace
            # (every workspace array starts 256-byte aligned)
            ws = p.g.ws_attn.view(torch.int32).cpu().numpy()
            order = next((ws[o:o + U] for o in range(0, ws.size - U + 1, 64)
                          if np.array_equal(np.sort(ws[o:o + U]), np.arange(U))), None)
            assert order is not None, "no dispatch order in the attention workspace"
            st = np_(p.g.tier_state).reshape(-1, 4)
            pages = (st[:, 2] + st[:, 3])[order]
            assert np.all(np.diff(pages) <= 0), pages
        seq = seq + 1
    check_pool_invariants(orc, p.o)


def test_decode_step_deferred_scores(dk, orc):
    """diffkv_decode_step(update_scores = 2) keeps the logits for a later
    diffkv_update_scores (one split per unit, where the step otherwise runs
    fused with the score update): the pair equals the oracle's step and
    attention with the score update, and the second call adds nothing twice."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", num_kv_heads=3, batch=5, max_seq_len=420, window=64)
    assert dk.diffkv_attn_splits(cfg, 5) == 1
    lens = torch.tensor([300, 41, 129, 77, 64], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) + 2 for n in lens) * 3 * 1.2) + 8
    p = Pair(dk, orc, cfg, 5, P, int(cu[-1]))
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    off = -(-dk.diffkv_workspace_bytes(cfg, dk.STEP, 5) // 256) * 256
    for step in range(3):
        dec = synth.make_decode(cfg, step)
        kn, vn, q = dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy()
        p.o.compact_step(seq, kn, vn)
        out_o = p.o.decode_attn(q, seq, update_scores=True)
        seq_d = torch.from_numpy(seq).to(dev)
        out_g = p.g.decode_step(torch.from_numpy(q).to(dev), seq_d, torch.from_numpy(kn).to(dev),
                                torch.from_numpy(vn).to(dev), update_scores=2)
        dk.diffkv_update_scores(cfg, p.g.pool, 5, p.g.page_table, p.g.tier_state, seq_d, p.g.ws_decode[off:])
        torch.cuda.synchronize()
        what = f"deferred decode step {step}"
        assert_state_equal(p.g, p.o, pages=False, what=what)
        assert_attn_close(out_g, out_o, what)
        assert_scores_close(p.g, p.o, what)
        resync_scores(p.g, p.o)
        seq = seq + 1


def test_decode_step_exhausted_pool(dk, orc):
    """A step that cannot get its page commits nothing; the attention still
    runs on the unchanged cache (as the two separate calls would)."""
    cfg = dict(head_dim=64, num_kv_heads=1, gqa_group=2, max_seq_len=100, window=64,
               alpha_h=1.0, alpha_l=0.2)
    rng = np.random.default_rng(6)
    N = 32
    k = rng.standard_normal((N, 1, 64)).astype(np.float16).view(np.uint16)
    sc = np.zeros((1, N), np.float32)
    p = Pair(dk, orc, cfg, 1, 2, N)
    p.prompt(np.array([0, N]), k, k, sc)
    kn = k[:1].reshape(1, 1, 64).copy()
    q = rng.standard_normal((1, 2, 64)).astype(np.float16).view(np.uint16)
    p.decode_step(np.array([N], np.int32), kn, kn, q, True, "exhausted decode step")
    assert int(p.o.status[0]) == orc.ST_POOL_EXHAUSTED


def _plan_record_words(g, cfg):
    """The plan-record magic of every unit's first page (0 where none)."""
    from tests.parity import plan_record_span
    off, _ = plan_record_span(cfg)
    first = g.page_table[..., 0].reshape(-1).to(torch.int64)
    pages = g.pool.pages.view(g.pool.num_pages, -1)
    ok = first >= 0
    idx = first.clamp(min=0)
    w = pages[idx][:, off:off + 4].contiguous().view(torch.int32).reshape(-1)
    return torch.where(ok, w, torch.zeros_like(w))


def _assert_caches_equal(a_, b_, P, what):
    """Two caches byte-identical: table, tier state, pool lists and pointer, pages."""
    for name in ("page_table", "tier_state"):
        assert torch.equal(getattr(a_, name), getattr(b_, name)), f"{what}: {name} differs"
    assert torch.equal(a_.pool.free_list, b_.pool.free_list), f"{what}: free lists differ"
    assert torch.equal(a_.pool.ptr, b_.pool.ptr), f"{what}: pointers differ"
    pa, pb = np_(a_.pool.pages.view(P, -1)), np_(b_.pool.pages.view(P, -1))
    live = sorted({int(x) for x in np_(a_.page_table).ravel() if x >= 0})
    bad = [p_ for p_ in live if not np.array_equal(pa[p_], pb[p_])]
    assert not bad, f"{what}: {len(bad)} of {len(live)} live pages differ, first {bad[:5]}"


def _twin_caches(dk, cfg, batch, lens, P, n):
    from workloads import synth
    pr = synth.make_prompt(cfg, lens=lens)
    st = []
    for _ in range(n):
        s_ = dk.DiffKVState(cfg, batch, P, max_total_tokens=int(lens.sum()), device=dev)
        cu = pr["cu_seqlens"].to(dev)
        tiers, _ = s_.classify(cu, pr["scores"].to(dev))
        s_.compact_prompt(cu, pr["k"].to(dev), pr["v"].to(dev), pr["scores"].to(dev), tiers)
        st.append(s_)
    return st


@pytest.mark.parametrize("batch", [32, 64])
def test_plan_record_matches_scan(dk, orc, batch):
    """The next step's plan that the fused score update leaves behind gives
    exactly the state a fresh scan gives: three identical caches -- A steps
    chained (plans from the previous step's workspace slot, no plan kernel),
    B through the plan kernel reading the records in each unit's first page,
    C through the plan kernel with every record erased before each step (a
    scan) -- stay byte-identical."""
    from tests.parity import plan_record_span, first_pages, masked
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", batch=batch, max_seq_len=1500)
    assert dk.diffkv_attn_splits(cfg, batch) == 1
    g = torch.Generator().manual_seed(51)
    lens = (torch.randint(5, 80, (batch,), generator=g) * 16 -
            torch.randint(0, 3, (batch,), generator=g)).to(torch.int64)
    P = int(sum(-(-int(n) // 16) for n in lens) * 8 * 1.2) + 64
    st = _twin_caches(dk, cfg, batch, lens, P, 3)
    off, n = plan_record_span(cfg)
    seq = lens.to(torch.int32).to(dev)
    used = 0
    for step in range(8):
        dec = synth.make_decode(cfg, step, device=dev)
        # cache C: erase every record, so its plan kernel scans
        c_ = st[2]
        first = c_.page_table[..., 0].reshape(-1)
        first = first[first >= 0].to(torch.int64)
        c_.pool.pages.view(c_.pool.num_pages, -1)[first, off:off + n] = 0
        used += int((_plan_record_words(st[1], cfg) != 0).sum())
        chains = (None, 0, 0)
        outs = [s_.decode_step(dec["q"], seq, dec["k_new"], dec["v_new"], update_scores=1, chain=c)
                for s_, c in zip(st, chains)]
        torch.cuda.synchronize()
        assert st[0].chain == step + 1
        assert torch.equal(outs[0], outs[1]), f"step {step}: outputs of A and B differ"
        assert torch.equal(outs[1], outs[2]), f"step {step}: outputs of B and C differ"
        _assert_caches_equal(st[0], st[1], P, f"step {step}: chained vs records")
        b_, c2 = st[1], st[2]
        for name in ("page_table", "tier_state"):
            assert torch.equal(getattr(b_, name), getattr(c2, name)), f"step {step}: {name} differs"
        assert torch.equal(b_.pool.free_list, c2.pool.free_list) and torch.equal(b_.pool.ptr, c2.pool.ptr)
        pb, pc = np_(b_.pool.pages.view(P, -1)), np_(c2.pool.pages.view(P, -1))
        fp = first_pages(np_(b_.page_table))
        for p_ in sorted({int(x) for x in np_(b_.page_table).ravel() if x >= 0}):
            x, y = (masked(pb[p_], cfg), masked(pc[p_], cfg)) if p_ in fp else (pb[p_], pc[p_])
            assert np.array_equal(x, y), f"step {step}: page {p_} differs"
        seq = seq + 1
    assert used > 0, "no plan record was used"
    for s_ in st:
        assert int(s_.pool.status.item()) == 0


@pytest.mark.parametrize("d,G,lo", [(128, 4, 1), (64, 5, 1), (128, 7, 0), (64, 16, 1)])
def test_split_plan_record_matches_scan(dk, orc, d, G, lo):
    """With several splits per unit the score update runs in 16-page chunks
    that leave candidates, from which a finishing kernel writes the next
    step's plan record.  Stepping from those records is byte-identical to
    stepping with every record erased before each step (the plan kernel then
    scans), over steps on units of very different sizes, and the records are
    used."""
    from tests.parity import first_pages, masked, plan_record_span
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", head_dim=d, gqa_group=G, lo_enabled=lo, num_kv_heads=3,
                      batch=5, max_seq_len=2100, window=64)
    assert dk.diffkv_attn_splits(cfg, 5) > 1
    lens = torch.tensor([2000, 37, 900, 1500, 300], dtype=torch.int64)
    P = int(sum(-(-int(n) // 16) + 2 for n in lens) * 3 * 1.2) + 8
    b_, c_ = _twin_caches(dk, cfg, 5, lens, P, 2)
    off, n = plan_record_span(cfg)
    seq = lens.to(torch.int32).to(dev)
    used = 0
    _say(f"split plan records d={d} G={G} lo={lo} splits={dk.diffkv_attn_splits(cfg, 5)}")
    for step in range(10):
        dec = synth.make_decode(cfg, step, device=dev)
        first = c_.page_table[..., 0].reshape(-1)
        first = first[first >= 0].to(torch.int64)
        c_.pool.pages.view(P, -1)[first, off:off + n] = 0
        used += int((_plan_record_words(b_, cfg) != 0).sum())
        ob = b_.decode_step(dec["q"], seq, dec["k_new"], dec["v_new"], update_scores=1)
        oc = c_.decode_step(dec["q"], seq, dec["k_new"], dec["v_new"], update_scores=1)
        torch.cuda.synchronize()
        assert torch.equal(ob, oc), f"step {step}: outputs differ"
        for name in ("page_table", "tier_state"):
            assert torch.equal(getattr(b_, name), getattr(c_, name)), f"step {step}: {name} differs"
        assert torch.equal(b_.pool.free_list, c_.pool.free_list) and torch.equal(b_.pool.ptr, c_.pool.ptr)
        pb, pc = np_(b_.pool.pages.view(P, -1)), np_(c_.pool.pages.view(P, -1))
        fp = first_pages(np_(b_.page_table))
        for p_ in sorted({int(x) for x in np_(b_.page_table).ravel() if x >= 0}):
            x, y = (masked(pb[p_], cfg), masked(pc[p_], cfg)) if p_ in fp else (pb[p_], pc[p_])
            assert np.array_equal(x, y), f"step {step}: page {p_} differs"
        seq = seq + 1
    assert used > 0, "no plan record was used"
    for s_ in (b_, c_):
        assert int(s_.pool.status.item()) == 0


@pytest.mark.parametrize("d,G,lo", [(128, 4, 1), (64, 5, 1), (128, 7, 0), (64, 16, 1)])
def test_chained_steps_match_plan_kernel(dk, orc, d, G, lo):
    """Chained decode steps (each planned by the previous step's attention)
    against the same steps through the plan kernel, for both head sizes,
    both weight-column layouts and the low tier off: outputs and caches
    byte-identical over steps that cross page boundaries, a release with
    re-admission in the middle (the chain restarts) and a step without the
    score update (which ends the chain)."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", head_dim=d, gqa_group=G, lo_enabled=lo, num_kv_heads=3,
                      batch=5, max_seq_len=420, window=64)
    assert dk.diffkv_attn_splits(cfg, 5) == 1
    lens = torch.tensor([383, 37, 200, 127, 64], dtype=torch.int64)
    P = int(sum(-(-int(n) // 16) + 2 for n in lens) * 3 * 1.2) + 8
    a_, b_ = _twin_caches(dk, cfg, 5, lens, P, 2)
    seq = lens.to(torch.int32)

    def both(step, upd=1):
        dec = synth.make_decode(cfg, step, device=dev)
        sd = seq.to(dev)
        oa = a_.decode_step(dec["q"], sd, dec["k_new"], dec["v_new"], update_scores=upd)
        ob = b_.decode_step(dec["q"], sd, dec["k_new"], dec["v_new"], update_scores=upd, chain=0)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"step {step}: outputs differ"
        _assert_caches_equal(a_, b_, P, f"step {step}")

    _say(f"chained steps d={d} G={G} lo={lo}")
    for step in range(12):
        both(step)
        seq = seq + 1
    assert a_.chain == 12
    mask = torch.tensor([1, 0, 0, 1, 0], dtype=torch.uint8, device=dev)
    a_.release(mask)
    b_.release(mask)
    lens2 = torch.tensor([95, 0, 0, 300, 0], dtype=torch.int64)
    pr2 = synth.make_prompt(cfg, lens=lens2, salt=5)
    for s_ in (a_, b_):
        cu = pr2["cu_seqlens"].to(dev)
        tiers, _ = s_.classify(cu, pr2["scores"].to(dev))
        s_.compact_prompt(cu, pr2["k"].to(dev), pr2["v"].to(dev), pr2["scores"].to(dev), tiers)
    assert a_.chain == 0
    seq = torch.where(mask.cpu() == 1, lens2.to(torch.int32), seq)
    for step in range(6):
        both(50 + step, upd=0 if step == 3 else 1)
        seq = seq + 1
    assert a_.chain == 2
    for s_ in (a_, b_):
        assert int(s_.pool.status.item()) == 0


def test_chain_broken_aborts_step(dk, orc):
    """A chained call on a cache that does not match the plans (the length
    not advanced; then a workspace overwritten with arbitrary words) aborts
    the whole step with STALE_CHAIN alone: nothing is committed and the
    attention runs on the unchanged cache, as an attention call alone would;
    repeated with chain = 0 the step commits and matches the plan kernel's."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", batch=32, max_seq_len=1500)
    g = torch.Generator().manual_seed(52)
    lens = (torch.randint(5, 80, (32,), generator=g) * 16 - torch.randint(0, 3, (32,), generator=g)).to(torch.int64)
    P = int(sum(-(-int(n) // 16) for n in lens) * 8 * 1.2) + 64
    a_, b_ = _twin_caches(dk, cfg, 32, lens, P, 2)
    seq = lens.to(torch.int32).to(dev)
    for step in range(3):
        dec = synth.make_decode(cfg, step, device=dev)
        for s_ in (a_, b_):
            s_.decode_step(dec["q"], seq, dec["k_new"], dec["v_new"], update_scores=1)
        seq = seq + 1
    torch.cuda.synchronize()
    _assert_caches_equal(a_, b_, P, "before the broken chain")
    # A: a chained call with the previous step's length; B: the attention alone
    dec = synth.make_decode(cfg, 3, device=dev)
    stale = seq - 1
    oa = a_.decode_step(dec["q"], stale, dec["k_new"], dec["v_new"], update_scores=1)
    ob = b_.decode_attn(dec["q"], stale, update_scores=1)
    torch.cuda.synchronize()
    assert int(a_.pool.status.item()) == dk.ST_STALE_CHAIN
    assert int(b_.pool.status.item()) == 0
    # (with no unit committing, the fused kernel's page order and arithmetic
    # are the attention kernel's)
    assert torch.equal(oa, ob), "broken chain: attention differs"
    _assert_caches_equal(a_, b_, P, "broken chain")
    # recovery: the status cleared, the step repeated without the chain
    a_.pool.status.zero_()
    for s_ in (a_, b_):
        s_.decode_step(dec["q"], seq, dec["k_new"], dec["v_new"], update_scores=1, chain=0)
    torch.cuda.synchronize()
    assert int(a_.pool.status.item()) == 0
    _assert_caches_equal(a_, b_, P, "recovered step")
    # a workspace overwritten with arbitrary words: the same abort, and no
    # other status bit (the words' own flag bits are not taken)
    seq = seq + 1
    dec = synth.make_decode(cfg, 4, device=dev)
    a_.ws_decode.fill_(0xFF)
    assert a_.chain > 0
    oa = a_.decode_step(dec["q"], seq, dec["k_new"], dec["v_new"], update_scores=1)
    ob = b_.decode_attn(dec["q"], seq, update_scores=1)
    torch.cuda.synchronize()
    assert int(a_.pool.status.item()) == dk.ST_STALE_CHAIN, hex(int(a_.pool.status.item()))
    assert torch.equal(oa, ob), "overwritten workspace: attention differs"
    _assert_caches_equal(a_, b_, P, "overwritten workspace")
    a_.pool.status.zero_()
    for s_ in (a_, b_):
        s_.decode_step(dec["q"], seq, dec["k_new"], dec["v_new"], update_scores=1, chain=0)
    torch.cuda.synchronize()
    assert int(a_.pool.status.item()) == 0
    _assert_caches_equal(a_, b_, P, "recovered after the overwrite")


def test_deterministic_replay(dk, orc):
    """Same inputs twice -> byte-identical state and outputs."""
    from workloads import synth
    cfg = _medium_cfg("llama3_8b", num_kv_heads=4, batch=3, max_seq_len=2000)
    lens = torch.tensor([1800, 333, 1024], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    res = []
    for _ in range(2):
        gst = dk.DiffKVState(cfg, 3, 2000, max_total_tokens=int(lens.sum()), device=dev)
        cu = pr["cu_seqlens"].to(dev)
        sc = pr["scores"].to(dev)
        tiers, _ = gst.classify(cu, sc)
        gst.compact_prompt(cu, pr["k"].to(dev), pr["v"].to(dev), sc, tiers)
        seq = lens.to(torch.int32).to(dev)
        outs = []
        for step in range(3):
            dec = synth.make_decode(cfg, step)
            gst.compact_step(seq, dec["k_new"].to(dev), dec["v_new"].to(dev))
            outs.append(np_(gst.decode_attn(dec["q"].to(dev), seq, update_scores=1)))
            seq = seq + 1
        torch.cuda.synchronize()
        live = sorted({int(x) for x in np_(gst.page_table).ravel() if x >= 0})
        res.append((np_(gst.page_table), np_(gst.pool.free_list), np_(gst.pool.pages.view(2000, -1))[live],
                    np.stack(outs)))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)
