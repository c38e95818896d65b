"""GPU parity of more than two precision levels (DiffKV notes, "KV
compression policy", extensibility paragraph; "Memory management",
generation workflow: extra levels through unidirectional or bidirectional
page tables) against the oracle: K = 3 and 4 levels through prompt
compaction, generation steps (every policy case: t_c kept, demoted to any
level or pruned; victims moving down one or more levels or pruned), release
and re-admission (tier state, both table rows, free list and every byte of
every live page bit-exact), decode attention with and without the score
update in one split per unit and in several, and the decode-step entry
(update_scores 0, 1 and 2 with diffkv_update_scores).  Tolerances are the
default codec's: attention 2e-3 + 1e-3 |ref|, score sums 1e-5 + 1e-4 |ref|."""
import numpy as np
import pytest
import torch

from tests.invariants import check_pool_invariants
from tests.parity import assert_attn_close, assert_scores_close, assert_state_equal, resync_scores
from tests.test_gpu_parity import Pair, _say

pytestmark = pytest.mark.gpu
dev = torch.device("cuda:0")


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


def _levels_cfg(K, **over):
    from workloads import synth
    c = synth.config("llama3_8b")
    c.pop("pool_factor", None)
    c.update(hi_k_bits=8, hi_v_bits=8, lo_k_bits=4, lo_v_bits=2, num_levels=K)
    if K == 3:
        c.update(alpha_h=1.0, alpha_mid=[0.85], alpha_l=0.75, mid_k_bits=[8], mid_v_bits=[2])
    else:
        c.update(alpha_h=1.0, alpha_mid=[0.9, 0.8], alpha_l=0.7, mid_k_bits=[8, 4], mid_v_bits=[4, 4])
    c.update(over)
    return c


CASES = [(3, 128, 4), (3, 64, 5), (4, 128, 8), (4, 64, 16), (3, 128, 7)]


@pytest.mark.parametrize("K,d,G", CASES)
def test_levels_ragged_prompt_steps_attention(dk, orc, K, d, G):
    """Ragged batch (tails inside pages, a prompt shorter than the window):
    prompt compaction, 24 steps each followed by attention (score update on
    every other step), release of half the batch, re-admission; the policy
    cases the oracle took are counted."""
    from workloads import synth
    cfg = _levels_cfg(K, head_dim=d, gqa_group=G, num_kv_heads=3, batch=5, max_seq_len=3000, window=16)
    assert dk.diffkv_page_bytes(cfg) == orc.page_bytes(cfg) > 0
    lens = torch.tensor([1500, 9, 700, 1201, 64], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 3 * 1.2) + 64
    p = Pair(dk, orc, cfg, 5, P, int(cu[-1]))
    _say(f"levels K={K} d={d} G={G}: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    check_pool_invariants(orc, p.o)
    seq = lens.numpy().astype(np.int32)
    cases = set()
    for step in range(24):
        dec = synth.make_decode(cfg, step)
        _say("  step", step)
        kn, vn = dec["k_new"].numpy(), dec["v_new"].numpy()
        br = p.o.copy().compact_step(seq, kn, vn, branches=True)
        cases |= {(int(x) & 15, (int(x) >> 4) & 15) for x in br.ravel() if x >= 0}
        p.step(seq, kn, vn, f"step {step}")
        q = (dec["q"].numpy().view(np.float16).astype(np.float32) * 3).astype(np.float16).view(np.uint16)
        p.attend(q, seq, step % 2 == 0, f"attn {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)
    _say("  cases", sorted(cases))
    assert (0, 0) in cases and (15, 15) in cases and any(c[0] >= 1 and c[0] < 14 for c in cases), cases
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


def test_levels_policy_cases_on_small_units(dk, orc):
    """Short prompts and a small window, 160 steps with sharp queries: every
    case of the K-level step occurs (t_c in each level and pruned; level-0
    victims to each lower level and pruned; lower victims moving further
    down and pruned), each step bit-exact against the oracle."""
    cfg = dict(head_dim=64, num_kv_heads=2, gqa_group=2, max_seq_len=700, window=6, alpha_h=1.0, alpha_l=0.7,
               num_levels=4, alpha_mid=[0.9, 0.8], mid_k_bits=[8, 4], mid_v_bits=[4, 4],
               hi_k_bits=8, hi_v_bits=8, lo_k_bits=4, lo_v_bits=2)
    rng = np.random.default_rng(0)
    d, H, G, B = 64, 2, 2, 2
    lens = np.array([40, 3])
    cu = np.concatenate([[0], np.cumsum(lens)])
    total = int(cu[-1])
    scale = np.ones(d, np.float32)
    scale[[3, 17]] = 8.0
    k = (rng.standard_normal((total, H, d)) * scale).astype(np.float16).view(np.uint16)
    v = (rng.standard_normal((total, H, d)) * scale).astype(np.float16).view(np.uint16)
    sc = (rng.random((H, total)) ** 4).astype(np.float32)
    sc /= sc.sum(1, keepdims=True) / 4
    p = Pair(dk, orc, cfg, B, 300, total)
    p.prompt(cu, k, v, sc)
    seq = lens.astype(np.int32).copy()
    cases = set()
    for step in range(160):
        kn = (rng.standard_normal((B, H, d)) * scale).astype(np.float16).view(np.uint16)
        vn = (rng.standard_normal((B, H, d)) * scale).astype(np.float16).view(np.uint16)
        br = p.o.copy().compact_step(seq, kn, vn, branches=True)
        cases |= {(int(x) & 15, (int(x) >> 4) & 15) for x in br.ravel() if x >= 0}
        p.step(seq, kn, vn, f"step {step}")
        q = (rng.standard_normal((B, H * G, d)) * 3).astype(np.float16).view(np.uint16)
        p.attend(q, seq, True, f"attn {step}")
        seq += 1
    _say("  cases", sorted(cases))
    want = {(0, 0), (0, 1), (0, 2), (0, 3), (14, 15)}
    assert want <= cases and any(c[0] >= 1 and c[0] < 14 and c[1] == 14 for c in cases), sorted(cases)
    check_pool_invariants(orc, p.o)


@pytest.mark.parametrize("K", [3, 4])
def test_levels_split_units(dk, orc, K):
    """Few long units: each unit's pages over several workgroups and the
    split merge (attention with and without the score update, then decode
    steps through the single entry point)."""
    from workloads import synth
    cfg = _levels_cfg(K, num_kv_heads=2, gqa_group=4, batch=2, max_seq_len=6000, window=64)
    assert dk.diffkv_attn_splits(cfg, 2) > 1
    lens = torch.tensor([5500, 2300], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 2 * 1.2) + 32
    p = Pair(dk, orc, cfg, 2, P, int(cu[-1]))
    _say(f"levels K={K}: split units")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    for step in range(4):
        dec = synth.make_decode(cfg, step)
        _say("  step", step)
        if step < 2:
            p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
            p.attend(dec["q"].numpy(), seq, step == 1, f"attn {step}")
        else:
            p.decode_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy(), step == 3,
                          f"decode step {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)


@pytest.mark.parametrize("update", [0, 1, 2])
def test_levels_decode_step_entry(dk, orc, update):
    """diffkv_decode_step with four levels (many units, one split each):
    the STEP then the attention; update_scores = 2 keeps the logits for
    diffkv_update_scores."""
    from workloads import synth
    batch, H = 32, 8
    cfg = _levels_cfg(4, num_kv_heads=H, batch=batch, max_seq_len=1300)
    assert dk.diffkv_attn_splits(cfg, batch) == 1
    g = torch.Generator().manual_seed(53)
    lens = (torch.randint(4, 70, (batch,), generator=g) * 16 - torch.randint(0, 2, (batch,), generator=g))
    lens = lens.to(torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * H * 1.2) + 64
    p = Pair(dk, orc, cfg, batch, P, int(cu[-1]))
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    off = -(-dk.diffkv_workspace_bytes(cfg, dk.STEP, batch) // 256) * 256
    for step in range(3):
        dec = synth.make_decode(cfg, step)
        kn, vn, q = dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy()
        _say("  levels decode step", step, "update", update)
        what = f"levels decode step {step}"
        if update < 2:
            p.decode_step(seq, kn, vn, q, update == 1, what)
        else:
            p.o.compact_step(seq, kn, vn)
            out_o = p.o.decode_attn(q, seq, update_scores=True)
            seq_d = torch.from_numpy(seq).to(dev)
            out_g = p.g.decode_step(torch.from_numpy(q).to(dev), seq_d, torch.from_numpy(kn).to(dev),
                                    torch.from_numpy(vn).to(dev), update_scores=2)
            dk.diffkv_update_scores(cfg, p.g.pool, batch, p.g.page_table, p.g.tier_state, seq_d,
                                    p.g.ws_decode[off:])
            torch.cuda.synchronize()
            assert_state_equal(p.g, p.o, pages=False, what=what)
            assert_attn_close(out_g, out_o, what)
            assert_scores_close(p.g, p.o, what)
            resync_scores(p.g, p.o)
        seq = seq + 1
    check_pool_invariants(orc, p.o)


@pytest.mark.parametrize("K,d,G", [(3, 128, 4), (4, 64, 5), (4, 128, 8)])
def test_levels_page_bounds_and_scores(dk, orc, K, d, G):
    """Per-page key bounds and page scores over K levels (every level's
    pages with its own codec and page size; scores over both table rows):
    bounds bit-exact, scores to the fixed-order fp32 bound, after prompt
    compaction (an inactive request) and again after 6 generation steps."""
    from tests.test_gpu_page_bounds import _compare
    from workloads import synth
    cfg = _levels_cfg(K, head_dim=d, gqa_group=G, num_kv_heads=3, batch=4, max_seq_len=2400, window=16)
    lens = torch.tensor([1300, 40, 777, 2000], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 3 * 1.2) + 64
    p = Pair(dk, orc, cfg, 4, P, int(cu[-1]))
    _say(f"levels bounds K={K} d={d} G={G}: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    seq[1] = 0                                   # an inactive request
    q = synth.make_decode(cfg, 0)["q"].numpy().view(np.uint16)
    n = _compare(p, orc, cfg, q, seq, f"K={K} d={d} G={G}")
    levels = {int(l) for b in (0, 2, 3) for h in range(3) for l, _, _ in p.o.unit_tokens(b, h)}
    assert levels == set(range(K)), levels      # pages of every level took part
    seq = lens.numpy().astype(np.int32)
    for step in range(6):
        dec = synth.make_decode(cfg, step)
        p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
        seq = seq + 1
    _compare(p, orc, cfg, q, seq, f"K={K} d={d} G={G} after steps")
    _say(f"  {n} live pages")


@pytest.mark.parametrize("rule", [0, 1])
def test_levels_per_head_thresholds_and_rule(dk, orc, rule):
    """Three levels with per-KV-head outer thresholds (alpha_h and alpha_l
    per head, the middle one shared) and both prompt rules (alpha/N, and
    alpha/i for the i-th token): classification, prompt compaction and 12
    steps with score updates, bit-exact."""
    from workloads import synth
    cfg = _levels_cfg(3, num_kv_heads=3, batch=4, max_seq_len=2500, window=16, prompt_rule=rule,
                      alpha_h_head=[1.0, 1.2, 0.9], alpha_l_head=[0.75, 0.6, 0.8], alpha_h=9.0, alpha_l=0.0)
    lens = torch.tensor([1200, 40, 900, 333], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 3 * 1.2) + 64
    p = Pair(dk, orc, cfg, 4, P, int(cu[-1]))
    _say(f"levels per head, rule {rule}: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    for step in range(12):
        dec = synth.make_decode(cfg, step)
        p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
        p.attend(dec["q"].numpy(), seq, True, f"attn {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)


def test_levels_noalloc_entry(dk, orc):
    """The allocation-free decode attention on a three-level cache equals the
    workspace entry point byte for byte (output and updated pages)."""
    from workloads import synth
    cfg = _levels_cfg(3, num_kv_heads=2, batch=3, max_seq_len=1200)
    lens = torch.tensor([900, 130, 511], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 2 * 1.2) + 32
    p = Pair(dk, orc, cfg, 3, P, int(cu[-1]))
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq_d = torch.from_numpy(lens.numpy().astype(np.int32)).to(dev)
    q = torch.from_numpy(synth.make_decode(cfg, 0)["q"].numpy()).to(dev)
    pages0 = p.g.pool.pages.clone()
    out_a = p.g.decode_attn(q, seq_d, update_scores=1)
    pages_a = p.g.pool.pages.clone()
    p.g.pool.pages.copy_(pages0)
    out_b = torch.empty_like(out_a)
    rc = dk.diffkv_decode_attn_noalloc(cfg, p.g.pool, 3, q, p.g.page_table, p.g.tier_state, seq_d, out_b, 1)
    assert rc == dk.DIFFKV_OK
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(pages_a, p.g.pool.pages)
