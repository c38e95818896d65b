"""The C-ABI library loads and exports every entry point include/diffkv.h
declares; host-only queries and argument validation work without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "diffkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(diffkv_\w+)\s*\(", src)))


def test_header_declares_entry_points():
    names = _declared()
    for n in ("diffkv_classify", "diffkv_compact", "diffkv_decode_attn", "diffkv_page_bytes",
              "diffkv_workspace_bytes", "diffkv_pool_init"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import compressed_paged_attention_amd as dk
    L = dk.lib()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing


def test_host_queries_and_validation():
    import compressed_paged_attention_amd as dk
    from workloads import synth
    c = synth.config("llama3_8b")
    assert dk.diffkv_page_bytes(c) == 3584
    assert dk.diffkv_page_bytes(dict(c, head_dim=64)) == 2048
    assert dk.diffkv_table_len(c) == -(-c["max_seq_len"] // 16) + 1
    assert dk.diffkv_page_bytes(dict(c, head_dim=96)) == -1
    assert dk.diffkv_page_bytes(dict(c, alpha_l=2.0)) == -1
    assert dk.diffkv_page_bytes(dict(c, hi_page_tokens=8)) == -1
    for op in (dk.PROMPT, dk.STEP, dk.RELEASE, dk.ATTN, dk.ATTN_SCORES):
        assert dk.diffkv_workspace_bytes(c, op, 32, 131072) > 0
    assert dk.diffkv_workspace_bytes(c, 99, 32, 0) == 0
    assert dk.diffkv_workspace_bytes(c, dk.ATTN_SCORES, 32) > dk.diffkv_workspace_bytes(c, dk.ATTN, 32)
    assert 1 <= dk.diffkv_attn_splits(c, 32) <= 64
    # invalid arguments are rejected on the host, before any launch
    L = dk.lib()
    bad = dk.make_config(dict(c, head_dim=96))
    assert L.diffkv_classify(ctypes.byref(bad), 1, 0, None, None, None, None, None) == dk.DIFFKV_E_INVALID
    good = dk.make_config(c)
    pool = dk.diffkv_pool(None, None, None, None, 10, 3584)
    assert L.diffkv_compact(ctypes.byref(good), ctypes.byref(pool), dk.PROMPT, 1, 0, None, None, None, None,
                            None, None, None, None, None, None, 0, None) == dk.DIFFKV_E_INVALID
    assert L.diffkv_decode_attn(ctypes.byref(good), ctypes.byref(pool), 1, None, None, None, None, None, 0,
                                None, 0, None) == dk.DIFFKV_E_INVALID


def test_decode_step_host_validation():
    """diffkv_decode_step refuses a negative chain count and a workspace off
    256-byte alignment on the host (batch 0: no kernel could run either way);
    its workspace holds two step slots around the attention's."""
    import compressed_paged_attention_amd as dk
    from workloads import synth
    c = synth.config("llama3_8b")
    L = dk.lib()
    cfg = dk.make_config(c)
    fake = 1 << 20  # never dereferenced on the host
    pool = dk.diffkv_pool(fake, fake, fake, fake, 10, 3584)
    need = dk.diffkv_workspace_bytes(c, dk.DECODE_STEP_SCORES, 0)
    args = [ctypes.byref(cfg), ctypes.byref(pool), 0] + [fake] * 7
    assert L.diffkv_decode_step(*args, 1, -1, fake, need, None) == dk.DIFFKV_E_INVALID
    assert L.diffkv_decode_step(*args, 1, 0, fake + 16, need, None) == dk.DIFFKV_E_WORKSPACE
    assert L.diffkv_decode_step(*args, 1, 0, fake, need - 1, None) == dk.DIFFKV_E_WORKSPACE
    assert L.diffkv_decode_step(*args, 1, 3, fake, need, None) == dk.DIFFKV_OK
    for b in (1, 32, 300):
        step = dk.diffkv_workspace_bytes(c, dk.STEP, b)
        att = dk.diffkv_workspace_bytes(c, dk.ATTN_SCORES, b)
        r = lambda x: -(-x // 256) * 256
        assert dk.diffkv_workspace_bytes(c, dk.DECODE_STEP_SCORES, b) == r(step) + r(att) + step


def test_policy_and_bounds_host_validation():
    """The policy fields are checked with the config (prompt_rule 0 or 1;
    both per-head arrays or neither), and diffkv_page_scores refuses a query
    or bounds pointer its paired loads cannot use (batch 0: nothing would
    run either way)."""
    import compressed_paged_attention_amd as dk
    from workloads import synth
    c = synth.config("llama3_8b")
    L = dk.lib()
    assert dk.diffkv_page_bytes(dict(c, prompt_rule=1)) == 3584
    assert dk.diffkv_page_bytes(dict(c, prompt_rule=2)) == -1
    fake = 1 << 20  # never dereferenced on the host
    one = dk.make_config(c)
    one.alpha_h_head = fake
    assert L.diffkv_page_bytes(ctypes.byref(one)) == -1
    one.alpha_l_head = fake
    assert L.diffkv_page_bytes(ctypes.byref(one)) == 3584
    cfg = dk.make_config(c)
    pool = dk.diffkv_pool(fake, fake, fake, fake, 10, 3584)
    ok = [fake] * 6  # q, page_table, tier_state, seq_len, bounds, scores
    assert L.diffkv_page_scores(ctypes.byref(cfg), ctypes.byref(pool), 0, *ok, None) == dk.DIFFKV_OK
    for bad in ([fake + 2] + [fake] * 5, [fake] * 4 + [fake + 4, fake]):
        assert L.diffkv_page_scores(ctypes.byref(cfg), ctypes.byref(pool), 0, *bad, None) == dk.DIFFKV_E_INVALID


def test_codec_variant_page_bytes_and_validation():
    """Tier codec variants: the library's page size is the plain layout's
    (the larger tier: six 16-byte aligned segments, codes T d b / 8 bytes),
    the same as the oracle's for every width pair; widths outside
    {1, 2, 4, 8}, or some but not all four set, are refused; all four zero
    is the default layout."""
    import itertools

    import compressed_paged_attention_amd as dk
    import oracle
    from workloads import synth
    c = synth.config("llama3_8b")
    r16 = lambda x: -(-x // 16) * 16
    for d in (64, 128):
        for hk, hv, lk, lv in itertools.product((1, 2, 4, 8), repeat=4):
            v = dict(c, head_dim=d, hi_k_bits=hk, hi_v_bits=hv, lo_k_bits=lk, lo_v_bits=lv)
            want = max(r16(T * d * kb // 8) + r16(T * d * vb // 8) + 16 * T
                       for T, kb, vb in ((16, hk, hv), (32, lk, lv)))
            assert dk.diffkv_page_bytes(v) == want == oracle.page_bytes(v), (d, hk, hv, lk, lv)
            for op in (dk.ATTN, dk.ATTN_SCORES, dk.DECODE_STEP_SCORES):
                assert dk.diffkv_workspace_bytes(v, op, 4, 0) > 0
    assert dk.diffkv_page_bytes(dict(c, hi_k_bits=3, hi_v_bits=4, lo_k_bits=4, lo_v_bits=2)) == -1
    assert dk.diffkv_page_bytes(dict(c, hi_k_bits=8)) == -1
    assert dk.diffkv_page_bytes(dict(c, hi_k_bits=0, hi_v_bits=0, lo_k_bits=0, lo_v_bits=0)) == 3584
