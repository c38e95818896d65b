"""Pins of the oracle's prompt-phase importance (CPU).

DiffKV notes, "KV compression policy", prompt phase: the importance of a
token is the mean of the attention scores it receives from the tokens after
it in the prompt; the scores of the q heads sharing a KV head are combined
with max.  Reading taken (A4/A5): causal softmax per q head, max over the
group per (query, key), mean over the N-1-i later queries (the token's own
query excluded); the last token has no later query and gets 0.
"""
import numpy as np
import pytest


def _cfg(d, H, G, N):
    return dict(head_dim=d, num_kv_heads=H, gqa_group=G, max_seq_len=N + 8, window=0, alpha_h=1.0,
                alpha_l=0.2)


def _numpy_importance(q, k, H, G):
    """q [N, H*G, d], k [N, H, d] float64 -> [H, N] by brute force."""
    N, _, d = q.shape
    out = np.zeros((H, N))
    for h in range(H):
        amax = np.zeros((N, N))
        for g in range(G):
            s = q[:, h * G + g] @ k[:, h].T / np.sqrt(d)       # [query, key]
            s[np.triu_indices(N, 1)] = -np.inf                  # causal: key <= query
            a = np.exp(s - s.max(1, keepdims=True))
            a /= a.sum(1, keepdims=True)
            amax = np.maximum(amax, a)
        for i in range(N):
            cnt = N - 1 - i
            out[h, i] = amax[i + 1:, i].sum() / cnt if cnt > 0 else 0.0
    return out


def test_equal_keys_harmonic_closed_form(orc):
    # every key equal: query j spreads 1/(j+1) over keys 0..j, so token i
    # receives (H_N - H_{i+1}) / (N - 1 - i) from the later queries, whatever
    # the queries and the group size
    rng = np.random.default_rng(1)
    d, H, G, N = 64, 2, 3, 37
    k = np.repeat(rng.standard_normal((1, H, d)), N, 0).astype(np.float16)
    q = rng.standard_normal((N, H * G, d)).astype(np.float16)
    sc = orc.importance_causal(_cfg(d, H, G, N), [0, N], q.view(np.uint16), k.view(np.uint16))
    for i in range(N):
        cnt = N - 1 - i
        ref = sum(1.0 / (j + 1) for j in range(i + 1, N)) / cnt if cnt else 0.0
        assert np.allclose(sc[:, i], ref, rtol=1e-6, atol=0)


def test_matches_numpy_brute_force_ragged(orc):
    rng = np.random.default_rng(2)
    d, H, G = 64, 2, 3
    lens = [23, 1, 40]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = (rng.standard_normal((cu[-1], H * G, d)) * 1.5).astype(np.float16)
    k = rng.standard_normal((cu[-1], H, d)).astype(np.float16)
    sc = orc.importance_causal(_cfg(d, H, G, max(lens)), cu, q.view(np.uint16), k.view(np.uint16))
    for r, n in enumerate(lens):
        a, b = cu[r], cu[r + 1]
        ref = _numpy_importance(q[a:b].astype(np.float64), k[a:b].astype(np.float64), H, G)
        assert np.allclose(sc[:, a:b], ref, rtol=1e-6, atol=1e-12)
    assert np.all(sc[:, cu[1:] - 1] == 0.0)       # last token of each prompt


def test_group_max_worked_case(orc):
    # head 0 puts (all but e^-48 of) its weight on token 0 from every query;
    # head 1 has a zero query, so query j spreads exactly 1/(j+1).  Token 0
    # therefore receives 1.0 from every later query (max), the others the
    # harmonic mean of head 1 -- a sum over the group would give token 0
    # 1 + H and a mean half of each.
    d, N = 64, 12
    k = -np.ones((N, 1, d), np.float16)
    k[0] = 1.0
    q = np.zeros((N, 2, d), np.float16)
    q[:, 0] = 3.0
    sc = orc.importance_causal(_cfg(d, 1, 2, N), [0, N], q.view(np.uint16), k.view(np.uint16))[0]
    assert sc[0] == np.float32(1.0)
    for i in range(1, N - 1):
        ref = sum(1.0 / (j + 1) for j in range(i + 1, N)) / (N - 1 - i)
        assert abs(sc[i] - ref) <= 1e-6 * ref


def test_equals_decode_score_updates_over_growing_prefixes(orc):
    # The decode-side score update (pinned separately) adds, for a query at
    # position j over a cache of tokens 0..j, max over the group of each
    # earlier token's weight.  Running it once per query of the prompt, each
    # time over a lossless cache of the prefix 0..j, accumulates exactly the
    # prompt importance times its count N-1-i.
    from tests.test_oracle_attention import _grid_token
    rng = np.random.default_rng(3)
    d, G, N = 64, 2, 18
    xk = np.stack([_grid_token(rng, d, 8, 4)[0] for _ in range(N)])
    xv = np.stack([_grid_token(rng, d, 8, 4)[1] for _ in range(N)])
    q = rng.standard_normal((N, G, d)).astype(np.float16)
    imp = orc.importance_causal(_cfg(d, 1, G, N), [0, N], q.view(np.uint16),
                                xk.astype(np.float16).view(np.uint16)[:, None, :])[0]
    got = np.zeros(N)
    for j in range(1, N):
        cfg = _cfg(d, 1, G, j + 1)
        st = orc.State(cfg, batch=1, num_pages=8)
        kk = xk[:j + 1].astype(np.float16).view(np.uint16)[:, None, :]
        vv = xv[:j + 1].astype(np.float16).view(np.uint16)[:, None, :]
        st.compact_prompt([0, j + 1], kk, vv, np.zeros((1, j + 1), np.float32),
                          np.full((1, j + 1), orc.HI, np.uint8))
        st.decode_attn(q[j:j + 1].view(np.uint16), [j], update_scores=True)
        for _, _, rec in st.unit_tokens(0, 0):
            got[rec["pos"]] += rec["score"]
    cnt = N - 1 - np.arange(N)
    assert np.allclose(got[:-1], imp[:-1].astype(np.float64) * cnt[:-1], rtol=2e-6)


def test_tail_equals_full_on_the_tail(orc):
    # the sampled variant gives the last tokens exactly the full values
    rng = np.random.default_rng(4)
    d, H, G = 64, 2, 2
    lens = [50, 9, 33]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((cu[-1], H * G, d)).astype(np.float16).view(np.uint16)
    k = rng.standard_normal((cu[-1], H, d)).astype(np.float16).view(np.uint16)
    cfg = _cfg(d, H, G, 64)
    full = orc.importance_causal(cfg, cu, q, k)
    part = orc.importance_causal(cfg, cu, q, k, tail=12)
    for r, n in enumerate(lens):
        a, b = cu[r], cu[r + 1]
        t = min(12, n)
        assert np.array_equal(part[:, b - t:b], full[:, b - t:b])
        assert np.all(part[:, a:b - t] == 0.0)
