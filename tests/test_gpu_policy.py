"""Policy variants on the device against the oracle ("KV compression
policy": the prompt-phase paragraph's alpha/i threshold for the i-th token;
the extensibility paragraph's per-head thresholds).

Every place that classifies is covered: the prompt classifier, the plan
kernel of a generation step, the plan a split attention's finishing kernel
records, and the plan the fused single-split attention records for a chained
step.  Tiers, counts and caches are compared bit for bit, attention within
the tolerances of the other parity tests.
"""
import numpy as np
import pytest
import torch

from tests.invariants import check_pool_invariants
from tests.test_gpu_parity import Pair, _say, dev

pytestmark = pytest.mark.gpu


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


AH, AL = [0.5, 1.0, 2.5], [0.1, 0.3, 0.6]


def _policy_cfg(d, G, lo, rule, per_head, **over):
    from workloads import synth
    cfg = synth.config("llama3_8b", head_dim=d, gqa_group=G, lo_enabled=lo, num_kv_heads=3, batch=5, **over)
    cfg.pop("pool_factor")
    cfg["prompt_rule"] = rule
    if per_head:
        cfg.update(alpha_h_head=AH, alpha_l_head=AL if lo else [0.2, 0.05, 0.6])
    return cfg


@pytest.mark.parametrize("lo", [1, 0])
@pytest.mark.parametrize("rule,per_head", [(1, False), (0, True), (1, True)])
def test_classify_policy_variants(dk, orc, rule, per_head, lo):
    """Prompt classification of ragged requests (lengths 0 to 3000) with sharp
    scores, so that all three tiers occur under every rule."""
    cfg = _policy_cfg(128, 4, lo, rule, per_head, max_seq_len=4096, window=16)
    rng = np.random.default_rng(40 + rule + 2 * per_head + 4 * lo)
    lens = np.array([3000, 0, 17, 1024, 333])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    H, total = 3, int(cu[-1])
    sc = np.empty((H, total), np.float32)
    for r, n in enumerate(lens):
        if n:
            x = rng.random((H, n)) ** 6
            sc[:, cu[r]:cu[r + 1]] = (x / x.sum(1, keepdims=True) * rng.uniform(0.3, 3.0, (H, 1)))
    tiers_o, counts_o = orc.classify(cfg, cu, sc)
    g = dk.DiffKVState(cfg, 5, 16, max_total_tokens=total, device=dev)
    tiers, counts = g.classify(torch.from_numpy(cu).to(dev), torch.from_numpy(sc).to(dev))
    torch.cuda.synchronize()
    t = tiers.cpu().numpy()
    assert np.array_equal(t, tiers_o) and np.array_equal(counts.cpu().numpy(), counts_o)
    for tier in (0, 2) + ((1,) if lo else ()):
        assert np.any(t == tier), f"tier {tier} never chosen"
    if per_head:        # the heads' pairs do change the outcome
        plain = orc.classify(dict(cfg, alpha_h_head=None, alpha_l_head=None), cu, sc)[0]
        assert not np.array_equal(plain, tiers_o)


@pytest.mark.parametrize("d,G,lo", [(128, 4, 1), (64, 16, 1), (128, 7, 0)])
def test_split_path_policy_variants(dk, orc, d, G, lo):
    """Long rows (several splits per unit): prompt with alpha/i and per-head
    pairs, then generation steps through diffkv_compact (plan kernel) with
    attention and the score update (finishing kernel records the next plan),
    then diffkv_decode_step on the recorded plans."""
    from workloads import synth
    cfg = _policy_cfg(d, G, lo, 1, True, max_seq_len=2100, window=32)
    assert dk.diffkv_attn_splits(cfg, 5) > 1
    lens = torch.tensor([2000, 37, 900, 1500, 300], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) + 2 for n in lens) * 3 * 1.2) + 8
    p = Pair(dk, orc, cfg, 5, P, int(cu[-1]))
    _say(f"policy split path d={d} G={G} lo={lo}: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    for step in range(5):
        dec = synth.make_decode(cfg, step, q_scale=3.0)
        _say("  step", step)
        p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
        p.attend(dec["q"].numpy(), seq, True, f"attn {step}")
        seq = seq + 1
    for step in range(5, 10):
        dec = synth.make_decode(cfg, step, q_scale=3.0)
        _say("  decode step", step)
        p.decode_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy(), True,
                      f"decode step {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)


@pytest.mark.parametrize("d,G,lo", [(128, 4, 1), (64, 5, 1), (128, 8, 0)])
def test_chained_policy_variants(dk, orc, d, G, lo):
    """Chained decode steps (each planned by the fused attention of the step
    before) with alpha/i prompts and per-head pairs: every step bit-exact
    with the oracle, and the heads take different policy cases."""
    from tests.test_gpu_chained import run_chained
    cfg = _policy_cfg(d, G, lo, 1, True, max_seq_len=480, window=8)
    lens = torch.tensor([383, 37, 20, 127, 14], dtype=torch.int64)
    acc = run_chained(dk, orc, cfg, lens, 48, 3.0, f"policy chained d={d} G={G} lo={lo}")
    assert acc["case"][2] > 0 and acc["case"][7] > 0
