"""GPU per-page key bounds and page scores (diffkv_page_bounds,
diffkv_page_scores) against the oracle.  Bounds: bit-exact (min/max of the
same dequantized fp32 keys).  Scores: the device multiplies in fp32 and sums
in a fixed order, the oracle in fp64: |gpu - ref| <= 1e-5 * sum_i
|max(q_i kmin_i, q_i kmax_i)| (plus 1e-30), the sum of the absolute terms
bounding the rounding of a sum of 64..128 terms; the page the device ranks
first is one whose exact score is within that bound of the maximum."""
import numpy as np
import pytest
import torch

from tests.test_gpu_parity import Pair

pytestmark = pytest.mark.gpu
dev = torch.device("cuda:0")


def _compare(p, orc, cfg, q, seq, what):
    bg = p.g.page_bounds()
    bo = p.o.page_bounds()
    live = ~np.isnan(bo[:, 0, 0])
    assert live.sum() > 0
    bgn = bg.cpu().numpy()
    assert np.array_equal(bgn[live], bo[live]), f"{what}: bounds differ"
    sg = p.g.page_scores(torch.from_numpy(q).to(dev), torch.from_numpy(seq).to(dev), bg).cpu().numpy()
    so = p.o.page_scores(q, seq, bo)
    assert np.array_equal(np.isneginf(sg), np.isneginf(so)), f"{what}: empty entries differ"
    H, G, d, L = cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"], so.shape[-1]
    fin = np.isfinite(so)
    # error scale per entry: sum of the absolute terms (max over the group)
    scale = np.zeros_like(so, dtype=np.float64)
    for b in range(so.shape[0]):
        for h in range(H):
            for t in np.flatnonzero(fin[b, h]):
                pid = int(p.o.page_table[b, h, t])
                mn, mx = bo[pid, 0].astype(np.float64), bo[pid, 1].astype(np.float64)
                qs = q[b, h * G:(h + 1) * G].view(np.float16).astype(np.float64)
                scale[b, h, t] = np.abs(np.maximum(qs * mn, qs * mx)).sum(1).max()
    err = np.abs(sg[fin].astype(np.float64) - so[fin])
    assert np.all(err <= 1e-5 * scale[fin] + 1e-30), f"{what}: page scores beyond tolerance"
    # the top page per unit: the device's choice is within the bound of the best
    for b in range(so.shape[0]):
        for h in range(H):
            if not fin[b, h].any():
                continue
            tg = int(np.argmax(np.where(fin[b, h], sg[b, h], -np.inf)))
            assert so[b, h].max() - so[b, h, tg] <= 2e-5 * scale[b, h].max()
    return int(live.sum())


@pytest.mark.parametrize("d,G,lo", [(128, 4, 1), (64, 5, 1), (128, 7, 0), (64, 16, 1)])
def test_page_bounds_and_scores_ragged(d, G, lo):
    import compressed_paged_attention_amd as dk
    import oracle
    from workloads import synth
    cfg = synth.config("llama3_8b", head_dim=d, gqa_group=G, lo_enabled=lo, num_kv_heads=3, batch=5,
                       max_seq_len=3000, window=64)
    cfg.pop("pool_factor")
    lens = torch.tensor([1500, 37, 700, 1201, 64], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 3 * 1.1) + 8
    p = Pair(dk, oracle, cfg, 5, P, int(cu[-1]))
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    seq = lens.numpy().astype(np.int32)
    seq[3] = 0                                   # an inactive request
    q = synth.make_decode(cfg, 0)["q"].numpy().view(np.uint16)
    n = _compare(p, oracle, cfg, q, seq, f"d={d} G={G} lo={lo}")
    print(f"page bounds d={d} G={G} lo={lo}: {n} live pages", flush=True)
    # after generation steps that write, demote and prune: refreshed bounds
    seq = lens.numpy().astype(np.int32)
    for step in range(3):
        dec = synth.make_decode(cfg, step)
        p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), f"step {step}")
        seq = seq + 1
    _compare(p, oracle, cfg, q, seq, f"d={d} G={G} lo={lo} after steps")


def test_page_bounds_llama3_full_batch():
    import compressed_paged_attention_amd as dk
    import oracle
    from workloads import synth
    cfg = synth.config("llama3_8b")
    B = cfg["batch"]
    lens = synth.seq_lens(cfg)
    pr = synth.make_prompt(cfg, lens=lens)
    P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
    p = Pair(dk, oracle, cfg, B, P, int(lens.sum()))
    p.prompt(pr["cu_seqlens"].numpy(), pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy(), check=False)
    del pr
    seq = lens.numpy().astype(np.int32)
    q = synth.make_decode(cfg, 0)["q"].numpy().view(np.uint16)
    n = _compare(p, oracle, cfg, q, seq, "llama3_8b")
    print(f"page bounds llama3_8b: {n} live pages", flush=True)


def test_page_bounds_long_units():
    """Long units (32768- and 20000-token prompts, low thresholds: 560 to
    880 live pages per unit out of 2065 entries): the entries spread over
    several workgroups of a unit and several rounds of each wave; then
    one generation step and a refresh."""
    import compressed_paged_attention_amd as dk
    import oracle
    from workloads import synth
    cfg = synth.config("long", batch=2, num_kv_heads=2, alpha_h=0.1, alpha_l=0.005)
    cfg.pop("pool_factor")
    lens = torch.tensor([32768, 20000], dtype=torch.int64)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    P = int(sum(-(-int(n) // 16) for n in lens) * 2 * 1.1) + 8
    p = Pair(dk, oracle, cfg, 2, P, int(cu[-1]))
    p.prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy())
    ts = p.o.tier_state.reshape(-1, 4)
    assert (ts[:, 2] + ts[:, 3]).max() > 800
    seq = lens.numpy().astype(np.int32)
    q = synth.make_decode(cfg, 0)["q"].numpy().view(np.uint16)
    n = _compare(p, oracle, cfg, q, seq, "long units")
    print(f"page bounds long units: {n} live pages", flush=True)
    dec = synth.make_decode(cfg, 1)
    p.step(seq, dec["k_new"].numpy(), dec["v_new"].numpy(), "step")
    _compare(p, oracle, cfg, q, seq + 1, "long units after a step")
