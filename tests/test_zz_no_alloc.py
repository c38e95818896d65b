"""diffkv_decode_attn_noalloc (scratch in a fixed device array of the
library, for callers that cannot allocate) against diffkv_decode_attn with
a caller workspace, through the C-ABI: two identical caches, the same calls
on each, outputs and every page byte (score sums included) identical; two
calls in a row, the second on a smaller batch (another launch shape: several
splits per unit); a request beyond the array's size is refused before any
launch."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

dev = torch.device("cuda:0")


def _clone(dk, g, cfg, B, P, total):
    c = dk.DiffKVState(cfg, B, P, max_total_tokens=total, device=dev)
    for name in ("page_table", "tier_state"):
        getattr(c, name).copy_(getattr(g, name))
    for name in ("pages", "free_list", "ptr", "status"):
        getattr(c.pool, name).copy_(getattr(g.pool, name))
    torch.cuda.synchronize()
    return c


def test_noalloc_matches_workspace_entry_point():
    import compressed_paged_attention_amd as dk
    from workloads import synth
    cfg = synth.config("llama3_8b")
    B, H, G, d = cfg["batch"], cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    lens = synth.seq_lens(cfg)
    P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
    pr = synth.make_prompt(cfg, device=dev, lens=lens)
    a = dk.DiffKVState(cfg, B, P, max_total_tokens=int(lens.sum()), device=dev)
    cu = pr["cu_seqlens"].to(dev)
    tiers, _ = a.classify(cu, pr["scores"])
    a.compact_prompt(cu, pr["k"], pr["v"], pr["scores"], tiers)
    del pr, tiers
    b = _clone(dk, a, cfg, B, P, int(lens.sum()))
    seq = lens.to(torch.int32).to(dev)
    calls = [(B, 1, 0), (8, 1, 1), (8, 0, 2)]      # (batch, update_scores, decode-input salt)
    for batch, upd, salt in calls:
        assert dk.diffkv_workspace_bytes(cfg, dk.ATTN_SCORES if upd else dk.ATTN, batch) <= dk.NOALLOC_SCRATCH_BYTES
        q = synth.make_decode(cfg, salt, device=dev)["q"]
        out_a = torch.full((B, H * G, d), 7.0, dtype=torch.float32, device=dev)
        out_b = out_a.clone()
        ws = torch.empty(dk.diffkv_workspace_bytes(cfg, dk.ATTN_SCORES, batch), dtype=torch.uint8, device=dev)
        dk.diffkv_decode_attn(cfg, a.pool, batch, q, a.page_table, a.tier_state, seq, out_a, upd, ws)
        rc = dk.diffkv_decode_attn_noalloc(cfg, b.pool, batch, q, b.page_table, b.tier_state, seq, out_b, upd)
        assert rc == dk.DIFFKV_OK
        torch.cuda.synchronize()
        print(f"batch {batch} update {upd} splits {dk.diffkv_attn_splits(cfg, batch)}", flush=True)
        assert torch.equal(out_a, out_b), f"batch {batch}: outputs differ"
        assert torch.equal(a.pool.pages, b.pool.pages), f"batch {batch}: pages differ"
        assert int(a.pool.status.item()) == int(b.pool.status.item()) == 0
        assert np.isfinite(out_b[:batch].cpu().numpy()).all()
    # beyond the array: refused on the host, nothing launched
    big = synth.config("stress_gqa8")
    assert dk.diffkv_workspace_bytes(big, dk.ATTN_SCORES, big["batch"]) > dk.NOALLOC_SCRATCH_BYTES
    before = b.pool.pages.clone()
    rc = dk.diffkv_decode_attn_noalloc(big, b.pool, big["batch"], q, b.page_table, b.tier_state, seq, out_b, 1)
    assert rc == dk.DIFFKV_E_WORKSPACE
    # deferred score update (logits kept for a later call) is not offered
    rc = dk.diffkv_decode_attn_noalloc(cfg, b.pool, B, q, b.page_table, b.tier_state, seq, out_b, 2)
    assert rc == dk.DIFFKV_E_INVALID
    torch.cuda.synchronize()
    assert torch.equal(before, b.pool.pages)
