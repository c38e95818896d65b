"""GPU query-free importance (diffkv_keydiff_scores, KeyDiff anchor cosine)
against the oracle.  The device sums in fp32 (fixed order), the oracle in
fp64; on these inputs (cosines away from 1, so 1 - cos keeps its bits) the
scores agree within 1e-4 |ref| + 1e-9, and classification of the device's
scores is bit-exact on both sides."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
dev = torch.device("cuda:0")
RTOL, ATOL = 1e-4, 1e-9


def _close(g, o, what):
    err = np.abs(g.astype(np.float64) - o)
    tol = RTOL * np.abs(o) + ATOL
    assert np.all(err <= tol), f"{what}: worst ratio {(err / tol).max():.2f}"
    return float((err / tol).max())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("raw", [False, True])
def test_keydiff_ragged(d, raw):
    import compressed_paged_attention_amd as dk
    import oracle
    rng = np.random.default_rng(d + raw)
    H = 3
    lens = [1, 100, 700, 257, 256]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    k = (rng.standard_normal((cu[-1], H, d)) + 0.5).astype(np.float16)
    cfg = dict(head_dim=d, num_kv_heads=H, gqa_group=1, max_seq_len=1024, window=8, alpha_h=1.0, alpha_l=0.2)
    ref = oracle.keydiff_scores(cfg, cu, k.view(np.uint16), anchor_raw=raw)
    got = dk.keydiff_scores(cfg, torch.from_numpy(cu).to(dev), torch.from_numpy(k.view(np.int16)).to(dev),
                            anchor_raw=raw).cpu().numpy()
    r = _close(got, ref, f"d={d} raw={raw}")
    print(f"keydiff d={d} raw={raw}: worst error / tolerance {r:.3f}", flush=True)


def test_keydiff_two_directions_on_device():
    import compressed_paged_attention_amd as dk
    d, na, nb = 128, 300, 700
    k = np.zeros((na + nb, 1, d), np.float16)
    k[:na, 0, 3] = 2.0
    k[na:, 0, 40] = 3.0
    cfg = dict(head_dim=d, num_kv_heads=1, gqa_group=1, max_seq_len=2048, window=0, alpha_h=1.0, alpha_l=0.2)
    got = dk.keydiff_scores(cfg, torch.tensor([0, na + nb], dtype=torch.int64, device=dev),
                            torch.from_numpy(k.view(np.int16)).to(dev)).cpu().numpy()[0]
    r = np.hypot(na, nb)
    wa, wb = 1 - na / r, 1 - nb / r
    tot = na * wa + nb * wb
    assert np.allclose(got[:na], wa / tot, rtol=1e-5) and np.allclose(got[na:], wb / tot, rtol=1e-5)


def test_keydiff_llama3_shape_and_tiers():
    """The Llama3-8B prompt shape (B32, 4096 tokens, 8 KV heads): every score
    against the oracle; the tiers of the device's scores bit-exact on both
    sides, and where they differ from the oracle's scores' tiers, the
    oracle's score lies within the tolerance of a threshold."""
    import compressed_paged_attention_amd as dk
    import oracle
    from workloads import synth
    cfg = synth.config("llama3_8b")
    lens = synth.seq_lens(cfg)
    pr = synth.make_prompt(cfg, lens=lens)
    cu = pr["cu_seqlens"].numpy()
    ref = oracle.keydiff_scores(cfg, cu, pr["k"].numpy())
    got_t = dk.keydiff_scores(cfg, pr["cu_seqlens"].to(dev), pr["k"].to(dev))
    got = got_t.cpu().numpy()
    r = _close(got, ref, "llama3_8b keydiff")
    print(f"keydiff llama3_8b: worst error / tolerance {r:.3f}", flush=True)
    st = dk.DiffKVState(cfg, cfg["batch"], 1024, max_total_tokens=int(cu[-1]), device=dev)
    tiers_g, counts_g = st.classify(pr["cu_seqlens"].to(dev), got_t)
    tiers_o, counts_o = oracle.classify(cfg, cu, got)
    assert np.array_equal(tiers_g.cpu().numpy(), tiers_o) and np.array_equal(counts_g.cpu().numpy(), counts_o)
    tiers_r, _ = oracle.classify(cfg, cu, ref)
    N = int(lens[0])
    for h, t in np.argwhere(tiers_r != tiers_o):
        s = float(ref[h, t]) * N
        near = min(abs(s - cfg["alpha_h"]), abs(s - cfg["alpha_l"]))
        assert near <= (RTOL * abs(float(ref[h, t])) + ATOL) * N
    hi = (tiers_o == 2).mean()
    print(f"  tiers from key-only scores: high {hi:.3f}, low {(tiers_o == 1).mean():.3f}", flush=True)
