"""GPU parity of the tier codec variants (the bit-split ablation of the
DiffKV notes' Results: K and V code widths per tier from {1, 2, 4, 8}, plain
page layout) against the oracle, through every entry point that reads or
writes pages: prompt compaction, generation steps, release and re-admission
(tier state, tables, free list and every byte of every live page
bit-exact), decode attention with and without the score update, in one
split per unit and in several, the decode-step entry (update_scores 0, 1
and 2 with the later diffkv_update_scores) and the per-page key bounds.
Tolerances are those of the default codec: attention 2e-3 + 1e-3 |ref|,
score sums 1e-5 + 1e-4 |ref|, bounds bit-exact."""
import numpy as np
import pytest
import torch

from tests.invariants import check_pool_invariants
from tests.parity import assert_attn_close, assert_scores_close, assert_state_equal, resync_scores
from tests.test_gpu_page_bounds import _compare
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


def _codec_cfg(codec, **over):
    from workloads import synth
    hk, hv, lk, lv = codec
    c = synth.config("llama3_8b", **over)
    c.pop("pool_factor", None)
    c.update(hi_k_bits=hk, hi_v_bits=hv, lo_k_bits=lk, lo_v_bits=lv)
    return c


# (K high, V high, K low, V low); (8, 4, 4, 2) is the default pair in the plain layout
CASES = [((4, 8, 2, 4), 128, 4, 1), ((8, 2, 4, 1), 64, 5, 1), ((8, 4, 4, 2), 128, 8, 1),
         ((2, 1, 1, 2), 64, 16, 1), ((1, 1, 1, 1), 128, 7, 0), ((8, 8, 8, 8), 64, 2, 1)]


@pytest.mark.parametrize("codec,d,G,lo", CASES)
def test_codec_ragged_prompt_steps_attention(dk, orc, codec, d, G, lo):
    """Ragged batch (tails inside pages, a prompt shorter than the window):
    prompt compaction, 6 steps each followed by attention with the score
    update, the page bounds, release of half the batch and re-admission."""
    from workloads import synth
    cfg = _codec_cfg(codec, head_dim=d, gqa_group=G, lo_enabled=lo, num_kv_heads=3, batch=5,
                     max_seq_len=3000, window=64)
    assert dk.diffkv_page_bytes(cfg) == orc.page_bytes(cfg) > 0
    lens = torch.tensor([1500, 37, 700, 1201, 64], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 3 * 1.1) + 8
    p = Pair(dk, orc, cfg, 5, P, int(cu[-1]))
    _say(f"codec {codec} d={d} G={G} lo={lo}: prompt")
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    check_pool_invariants(orc, p.o)
    seq = lens.numpy().astype(np.int32)
    for step in range(6):
        dec = synth.make_decode(cfg, step)
        _say("  step", step)
        p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
        p.attend(dec["q"].numpy(), seq, step % 2 == 0, f"attn {step}")
        seq = seq + 1
    check_pool_invariants(orc, p.o)
    _say("  bounds")
    _compare(p, orc, cfg, synth.make_decode(cfg, 50)["q"].numpy(), seq, "codec bounds")
    mask = np.array([1, 0, 1, 0, 1], np.uint8)
    p.release(mask)
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


@pytest.mark.parametrize("codec", [(4, 8, 2, 4), (2, 4, 1, 2)])
def test_codec_split_units(dk, orc, codec):
    """Few long units: each unit's pages spread over several workgroups
    whose partials the split merge combines (attention with and without the
    score update, then decode steps through the single entry point)."""
    from workloads import synth
    cfg = _codec_cfg(codec, num_kv_heads=2, gqa_group=4, batch=2, max_seq_len=6000, window=64)
    assert dk.diffkv_attn_splits(cfg, 2) > 1
    lens = torch.tensor([5500, 2300], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 2 * 1.1) + 16
    p = Pair(dk, orc, cfg, 2, P, int(cu[-1]))
    _say(f"codec {codec}: split units")
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
def test_codec_decode_step_entry(dk, orc, update):
    """diffkv_decode_step on a codec variant (many units, one split each):
    the STEP then the attention; update_scores = 2 keeps the logits for
    diffkv_update_scores."""
    from workloads import synth
    batch, H = 32, 8
    cfg = _codec_cfg((4, 8, 2, 4), num_kv_heads=H, batch=batch, max_seq_len=1300)
    assert dk.diffkv_attn_splits(cfg, batch) == 1
    g = torch.Generator().manual_seed(47)
    lens = (torch.randint(4, 70, (batch,), generator=g) * 16 - torch.randint(0, 2, (batch,), generator=g))
    lens = lens.to(torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * H * 1.1) + 64
    p = Pair(dk, orc, cfg, batch, P, int(cu[-1]))
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    off = -(-dk.diffkv_workspace_bytes(cfg, dk.STEP, batch) // 256) * 256
    for step in range(3):
        dec = synth.make_decode(cfg, step)
        kn, vn, q = dec["k_new"].numpy(), dec["v_new"].numpy(), dec["q"].numpy()
        _say("  codec decode step", step, "update", update)
        what = f"codec decode step {step}"
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
