"""GPU prompt-phase importance (diffkv_importance) against the oracle.

DiffKV notes, "KV compression policy", prompt phase: importance = mean of the
attention a token receives from the tokens after it, max over the KV head's
q heads.  The device computes the logits in fp32 on the matrix units from
fp16 inputs (exact products, fp32 sums), the weights with the hardware
exp2/log2 (about one ulp) and the means in fp32; the oracle in fp64.  Bound:
a logit error of a few fp32 ulps of sum |q_e k_e| / sqrt(d) (<= ~1e-5 on
these N(0,1) inputs with x8 outlier channels) moves a weight by <= ~1e-5
relative, the exp2/log2 and the fp32 sums add ~1e-6: |gpu - ref| <= 1e-4 |ref|
+ 1e-9 (the absolute term covers weights below fp32's resolution next to
larger ones).  Tiers are integers decided from the scores: the oracle's
classification of the device's scores must equal the device's (bit-exact),
and where the device's tiers differ from those of the oracle's scores the
oracle's score must lie within the tolerance of a threshold.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
dev = torch.device("cuda:0")
RTOL, ATOL = 1e-4, 1e-9


def _close(g, o, what):
    err = np.abs(g.astype(np.float64) - o)
    tol = RTOL * np.abs(o) + ATOL
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} scores beyond tolerance, worst ratio {(err / tol).max():.2f}"
    return float((err / tol).max())


def _cfg(d, H, G, S):
    return dict(head_dim=d, num_kv_heads=H, gqa_group=G, max_seq_len=S, window=64, alpha_h=1.0, alpha_l=0.2)


@pytest.mark.parametrize("d,G", [(64, 1), (64, 3), (128, 4), (128, 8)])
def test_causal_importance_ragged(d, G):
    import compressed_paged_attention_amd as dk
    import oracle
    rng = np.random.default_rng(d + G)
    H = 2
    lens = [1, 17, 130, 300, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    sc = np.ones(d, np.float32)
    sc[rng.choice(d, 4, replace=False)] = 8.0
    q = (rng.standard_normal((T, H * G, d))).astype(np.float16)
    k = (rng.standard_normal((T, H, d)) * sc).astype(np.float16)
    cfg = _cfg(d, H, G, 512)
    ref = oracle.importance_causal(cfg, cu, q.view(np.uint16), k.view(np.uint16))
    got = dk.importance(cfg, torch.from_numpy(cu).to(dev), torch.from_numpy(q.view(np.int16)).to(dev),
                        torch.from_numpy(k.view(np.int16)).to(dev)).cpu().numpy()
    r = _close(got, ref, f"d={d} G={G}")
    assert np.all(got[:, cu[1:] - 1] == 0.0)
    print(f"causal importance d={d} G={G}: worst error / tolerance {r:.3f}", flush=True)


def test_equal_keys_and_group_max_on_device():
    import compressed_paged_attention_amd as dk
    d, N = 64, 200
    # equal keys: token i receives (H_N - H_{i+1}) / (N - 1 - i)
    rng = np.random.default_rng(5)
    k = np.repeat(rng.standard_normal((1, 1, d)), N, 0).astype(np.float16)
    q = rng.standard_normal((N, 3, d)).astype(np.float16)
    cfg = _cfg(d, 1, 3, 256)
    cu = torch.tensor([0, N], dtype=torch.int64, device=dev)
    got = dk.importance(cfg, cu, torch.from_numpy(q.view(np.int16)).to(dev),
                        torch.from_numpy(k.view(np.int16)).to(dev)).cpu().numpy()[0]
    hn = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, N + 1))])
    ref = np.array([(hn[N] - hn[i + 1]) / (N - 1 - i) if i < N - 1 else 0.0 for i in range(N)])
    _close(got[None], ref[None], "equal keys")
    # group max: head 0 gives token 0 all its weight, head 1 spreads 1/(j+1)
    k = -np.ones((N, 1, d), np.float16)
    k[0] = 1.0
    q = np.zeros((N, 2, d), np.float16)
    q[:, 0] = 3.0
    cfg = _cfg(d, 1, 2, 256)
    got = dk.importance(cfg, cu, torch.from_numpy(q.view(np.int16)).to(dev),
                        torch.from_numpy(k.view(np.int16)).to(dev)).cpu().numpy()[0]
    assert abs(got[0] - 1.0) <= 1e-6
    _close(got[1:-1][None], ref[1:-1][None], "group max")


def test_probe_importance_tiny_and_tiers():
    """The tiny workload's recipe (16 probe queries per request that see every
    token) on the device: scores within tolerance of the oracle's, tiers of
    the device's scores bit-exact on both sides, and tier differences from
    the oracle's scores only next to a threshold."""
    import compressed_paged_attention_amd as dk
    import oracle
    from workloads import synth
    cfg = synth.config("tiny")
    pr = synth.make_prompt(cfg)
    qp = synth.probe_queries(cfg)
    cu = pr["cu_seqlens"].numpy()
    ref = oracle.importance_from_queries(cfg, cu, pr["k"].numpy(), qp.numpy())
    got = dk.importance(cfg, pr["cu_seqlens"].to(dev), qp.to(dev), pr["k"].to(dev), nq=cfg["nprobe"])
    g = got.cpu().numpy()
    _close(g, ref, "probe")
    st = dk.DiffKVState(cfg, 1, 64, max_total_tokens=int(cu[-1]), device=dev)
    tiers_g, counts_g = st.classify(pr["cu_seqlens"].to(dev), got)
    tiers_o, counts_o = oracle.classify(cfg, cu, g)
    assert np.array_equal(tiers_g.cpu().numpy(), tiers_o) and np.array_equal(counts_g.cpu().numpy(), counts_o)
    tiers_r, _ = oracle.classify(cfg, cu, ref)
    diff = np.argwhere(tiers_r != tiers_o)
    N = int(cu[1])
    for h, t in diff:
        s = float(ref[h, t]) * N
        near = min(abs(s - cfg["alpha_h"]), abs(s - cfg["alpha_l"]))
        assert near <= (RTOL * abs(float(ref[h, t])) + ATOL) * N, f"tier differs away from a threshold ({h},{t})"


def test_causal_importance_llama3_shape_sampled():
    """Full Llama3-8B prompt shape (B32, 4096 tokens, 8 KV heads, GQA 4,
    d = 128) on the device; sampled outputs through the oracle: the last 512
    tokens of two (request, KV head) pairs, whose importance needs only the
    queries after them (each over its whole causal row of up to 4096 keys);
    the pair's q heads and key head are sliced out (a head's importance
    depends on nothing else)."""
    import time

    import compressed_paged_attention_amd as dk
    import oracle
    from workloads import synth
    cfg = synth.config("llama3_8b")
    H, G, d = cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    lens = synth.seq_lens(cfg)
    pr = synth.make_prompt(cfg, device=dev, lens=lens)
    gq = torch.Generator(device=dev)
    gq.manual_seed(synth.SEED_BASE + 777)
    q = (torch.randn(int(lens.sum()), H * G, d, generator=gq, device=dev)).to(torch.float16).view(torch.int16)
    cu = pr["cu_seqlens"].to(dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    got = dk.importance(cfg, cu, q, pr["k"])
    torch.cuda.synchronize()
    print(f"llama3_8b importance: {1e3 * (time.perf_counter() - t0):.2f} ms (incl. allocation)", flush=True)
    tail = 512
    for r, h in ((5, 3), (31, 7)):
        a, b = int(pr["cu_seqlens"][r]), int(pr["cu_seqlens"][r + 1])
        qs = q[a:b, h * G:(h + 1) * G].contiguous().cpu().numpy().view(np.uint16)
        ks = pr["k"][a:b, h:h + 1].contiguous().cpu().numpy().view(np.uint16)
        ref = oracle.importance_causal(dict(cfg, num_kv_heads=1), [0, b - a], qs, ks, tail=tail)[0]
        r_ = _close(got[h, b - tail:b].cpu().numpy()[None], ref[None, -tail:], f"llama3_8b sampled r={r} h={h}")
        print(f"  request {r} head {h}: last {tail} tokens, worst error / tolerance {r_:.3f}", flush=True)
