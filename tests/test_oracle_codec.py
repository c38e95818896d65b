"""Pins of the oracle's fp16 conversion, codec and page layout (CPU only).

Sources: DiffKV notes, "Background" (asymmetric quantization: Q = round((X -
z)/s), X^ = s Q + z per K/V vector) and "Memory management" (unified pages
with six segments).  The fp16 conversion is pinned against numpy's IEEE
binary16 conversion, a library routine independent of the oracle.
"""
import math

import numpy as np
import pytest


def test_f16_decode_all_bit_patterns(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_encode_matches_numpy(orc):
    rng = np.random.default_rng(1)
    xs = [rng.standard_normal(20000).astype(np.float32) * s for s in (1e-7, 1e-5, 1e-3, 1, 300, 3e4)]
    # every fp16 value, midpoints between neighbours (ties), and just around them
    allh = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = ((allh[:-1] + allh[1:]) / 2).astype(np.float32)
    edge = np.array([0.0, -0.0, 65504, 65519.99, 65520, 65536, 1e9, -1e9, np.inf, -np.inf,
                     2.0**-24, 2.0**-25, 3 * 2.0**-26, 2.0**-14, 2.0**-14 - 2.0**-25], np.float32)
    x = np.concatenate(xs + [mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.float32(1e9)), edge])
    got = orc.f32_to_f16(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f16_nan(orc):
    assert np.isnan(orc.f16_to_f32(orc.f32_to_f16(np.array([np.nan], np.float32))))[0]


@pytest.mark.parametrize("bits", [8, 4, 2, 1])
def test_codec_roundtrip_bound(orc, bits):
    rng = np.random.default_rng(bits)
    qmax = (1 << bits) - 1
    for trial in range(300):
        scale = 10.0 ** rng.uniform(-3, 3)
        x16 = (rng.standard_normal(128) * scale).astype(np.float16)
        if trial % 3 == 0:
            x16[rng.integers(0, 128, 2)] *= 8  # outlier channels
        x = x16.astype(np.float32)
        s16, z16, codes = orc.quantize(x, bits)
        s = float(np.uint16(s16).view(np.float16))
        z = float(np.uint16(z16).view(np.float16))
        assert z == float(x.min())  # the min of fp16 data is an fp16 value
        assert codes.max() <= qmax
        xh = np.array([orc.dequant(s16, z16, int(c)) for c in codes])
        rng_ = float(x.max()) - float(x.min())
        # half a step, plus what the fp16 rounding of the scale can move the top code
        bound = s / 2 * (1 + 1e-6) + qmax * abs(s - rng_ / qmax) + 1e-6 * abs(z)
        assert np.all(np.abs(xh - x) <= bound + 1e-12), (trial, np.abs(xh - x).max(), bound)
        assert codes[np.argmin(x)] == 0


def test_codec_worked_values(orc):
    # step 1, zero 0: ties go to even (0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 7.5 -> 8)
    s, z, c = orc.quantize(np.array([0, 0.5, 1.5, 2.5, 7.5, 15], np.float32), 4)
    assert s == 0x3C00 and z == 0
    assert c.tolist() == [0, 0, 2, 2, 8, 15]
    # 2-bit: [-1, 0, 1, 2] -> step 1, zero -1, codes 0..3, dequant exact
    s, z, c = orc.quantize(np.array([-1, 0, 1, 2], np.float32), 2)
    assert c.tolist() == [0, 1, 2, 3]
    assert [orc.dequant(s, z, int(k)) for k in c] == [-1.0, 0.0, 1.0, 2.0]
    # 8-bit with an exact fp16 step: range 25.5 -> step 0.1 is not exact in fp16,
    # range 255 * 2^-4 -> step 2^-4 is
    x = np.arange(256, dtype=np.float32) * np.float32(2.0**-4) - 3
    s, z, c = orc.quantize(x, 8)
    assert float(np.uint16(s).view(np.float16)) == 2.0**-4
    assert c.tolist() == list(range(256))
    assert np.array_equal(np.array([orc.dequant(s, z, int(k)) for k in c], np.float32), x)


@pytest.mark.parametrize("bits", [8, 4, 2, 1])
def test_codec_constant_vector(orc, bits):
    x = np.full(64, 1.375, np.float32)
    s, z, c = orc.quantize(x, bits)
    assert s == 0 and np.all(c == 0)
    assert orc.dequant(s, z, 0) == 1.375


def test_codec_requantize_from_fp32(orc):
    # requantization works on fp32 values that need not be fp16: the zero is
    # the fp16 rounding of the min, so codes stay clamped in range
    rng = np.random.default_rng(7)
    for _ in range(200):
        x = rng.standard_normal(128).astype(np.float32) * np.float32(1.0 + 1e-4)
        s, z, c = orc.quantize(x, 4)
        assert c.max() <= 15 and c.min() >= 0
        zf = float(np.uint16(z).view(np.float16))
        assert zf == float(np.float32(x.min()).astype(np.float16))


def test_layout_sizes_and_budget(orc):
    for d, pb in ((128, 3584), (64, 2048)):
        c = dict(head_dim=d, num_kv_heads=1, gqa_group=1, max_seq_len=64, window=0,
                 alpha_h=1.0, alpha_l=0.2)
        assert orc.page_bytes(c) == pb
        for tier, T, kb, vb in ((orc.HI, 16, 8, 4), (orc.LO, 32, 4, 2)):
            T_, seg = orc.tier_layout(c, tier)
            assert T_ == T
            assert np.all(seg % 16 == 0) and np.all(np.diff(seg) > 0)
            sizes = np.diff(seg)
            assert sizes.tolist() == [T * d * kb // 8, 4 * T, T * d * vb // 8, 4 * T, 4 * T, 4 * T]
            assert seg[6] <= pb
        # the high tier K8V4 costs 1.5 d + 16 bytes per token (codes, two fp16
        # scale/zero pairs, fp32 score, int32 position)
        _, seg = orc.tier_layout(c, orc.HI)
        assert seg[6] / 16 == 1.5 * d + 16


@pytest.mark.parametrize("d", [64, 128])
def test_layout_fields_tile_segments(orc, d):
    c = dict(head_dim=d, num_kv_heads=1, gqa_group=1, max_seq_len=64, window=0, alpha_h=1.0, alpha_l=0.2)
    for tier, T, kb, vb in ((orc.HI, 16, 8, 4), (orc.LO, 32, 4, 2)):
        _, seg = orc.tier_layout(c, tier)
        for fn, bits, lo, hi in ((orc.k_code_addr, kb, seg[0], seg[1]), (orc.v_code_addr, vb, seg[2], seg[3])):
            seen = set()
            for t in range(T):
                for j in range(d):
                    b, s = fn(c, tier, t, j)
                    assert lo <= b < hi and s % bits == 0 and s + bits <= 8
                    for bit in range(s, s + bits):
                        key = (b, bit)
                        assert key not in seen
                        seen.add(key)
            assert len(seen) == (hi - lo) * 8  # every bit of the segment is used once


def test_v_layout_lane_chunks(orc):
    # The token-vectorized V layout: 64 lane chunks of d/8 bytes; chunk
    # i + 16 q holds dim j = i + 16 nb for the 4 tokens 4q..4q+3 (high tier)
    c = dict(head_dim=128, num_kv_heads=1, gqa_group=1, max_seq_len=64, window=0, alpha_h=1.0, alpha_l=0.2)
    _, seg = orc.tier_layout(c, orc.HI)
    for t in range(16):
        for j in range(128):
            b, s = orc.v_code_addr(c, orc.HI, t, j)
            lane = (b - seg[2]) // 16
            assert lane == (j % 16) + 16 * (t // 4)
    # first word of chunk 0: dims 0 and 16, tokens 0..3
    got = {orc.v_code_addr(c, orc.HI, t, j) for t in range(4) for j in (0, 16)}
    assert got == {(seg[2] + 0, 0), (seg[2] + 2, 0), (seg[2] + 0, 4), (seg[2] + 2, 4),
                   (seg[2] + 1, 0), (seg[2] + 3, 0), (seg[2] + 1, 4), (seg[2] + 3, 4)}


def test_table_length_reading(orc):
    # A row of S_max / T_h entries is one short: S_max = 32, 17 high + 15 low
    # tokens need 2 + 1 pages; the row holds ceil(S_max/T_h) + 1.
    c = dict(head_dim=128, num_kv_heads=1, gqa_group=1, max_seq_len=32, window=0, alpha_h=1.0, alpha_l=0.2)
    assert orc.table_len(c) == 3
    assert math.ceil(17 / 16) + math.ceil(15 / 32) == 3 > 32 // 16
    # derived size check: int32 rows of S_max/T_h = 4096/16 entries for
    # 32 layers x 8 KV heads x 128 requests total 32 MiB
    assert 32 * 8 * 128 * (4096 // 16) * 4 == 32 * 2**20


# --- tier codec variants ("Results": the bit-split ablation, K4V8, K2V4,
# K8V2, K4V1 against K8V4 / K4V2): the plain layout, token-major codes
# packed from bit 0

VARIANTS = [(4, 8, 2, 4), (8, 2, 4, 1), (8, 4, 4, 2), (2, 1, 1, 2)]


def _vcfg(d, codec):
    hk, hv, lk, lv = codec
    return dict(head_dim=d, num_kv_heads=1, gqa_group=1, max_seq_len=64, window=0, alpha_h=1.0,
                alpha_l=0.2, hi_k_bits=hk, hi_v_bits=hv, lo_k_bits=lk, lo_v_bits=lv)


@pytest.mark.parametrize("codec", VARIANTS)
def test_variant_layout_sizes(orc, codec):
    # segments of T d b / 8 bytes for the codes (16-byte aligned), the page
    # the larger tier; e.g. K4V8 at d = 128: 16 x 64 + 16 x 128 code bytes
    for d in (64, 128):
        c = _vcfg(d, codec)
        pages = []
        for tier, T, kb, vb in ((orc.HI, 16, codec[0], codec[1]), (orc.LO, 32, codec[2], codec[3])):
            T_, seg = orc.tier_layout(c, tier)
            assert T_ == T
            r16 = lambda x: -(-x // 16) * 16
            assert np.diff(seg).tolist() == [r16(T * d * kb // 8), 4 * T, r16(T * d * vb // 8), 4 * T, 4 * T, 4 * T]
            pages.append(seg[6])
        assert orc.page_bytes(c) == max(pages)
    # K4V8 high (1024 + 2048 code bytes + 256) against K2V4 low (32 tokens:
    # 1024 + 2048 + 512): the low tier sets the page
    assert orc.page_bytes(_vcfg(128, (4, 8, 2, 4))) == 32 * 32 + 32 * 64 + 4 * 4 * 32
    for bad in ((3, 4, 4, 2), (8, 4, 4, 0), (16, 4, 4, 2)):
        assert orc.page_bytes(_vcfg(128, bad)) == -1


@pytest.mark.parametrize("codec", VARIANTS)
def test_variant_fields_tile_segments(orc, codec):
    # every (token, dim) code of a tier has its own bits, token-major from
    # bit 0: code (t, j) at bit (t d + j) b of its segment
    d = 64
    c = _vcfg(d, codec)
    for tier, T, kb, vb in ((orc.HI, 16, codec[0], codec[1]), (orc.LO, 32, codec[2], codec[3])):
        _, seg = orc.tier_layout(c, tier)
        for fn, bits, lo in ((orc.k_code_addr, kb, seg[0]), (orc.v_code_addr, vb, seg[2])):
            seen = set()
            for t in range(T):
                for j in range(d):
                    b, sh = fn(c, tier, t, j)
                    assert (b - lo) * 8 + sh == (t * d + j) * bits
                    seen.update((b, x) for x in range(sh, sh + bits))
            assert len(seen) == T * d * bits


@pytest.mark.parametrize("codec", VARIANTS)
def test_variant_prompt_codes_within_half_a_step(orc, codec):
    # a prompt compacted with a variant codec: every retained token's K and V
    # read back from its page lie within half a quantization step (plus the
    # fp16 rounding of the scale) of the input, at the tier's width
    rng = np.random.default_rng(sum(codec))
    d, H, N = 64, 2, 100
    c = dict(_vcfg(d, codec), num_kv_heads=H, max_seq_len=256, window=8)
    cu = np.array([0, N])
    k = rng.standard_normal((N, H, d)).astype(np.float16)
    v = rng.standard_normal((N, H, d)).astype(np.float16)
    sc = (rng.random((H, N)) ** 3 / 20).astype(np.float32)
    tiers, counts = orc.classify(c, cu, sc)
    st = orc.State(c, batch=1, num_pages=64)
    st.compact_prompt(cu, k.view(np.uint16), v.view(np.uint16), sc, tiers)
    widths = {orc.HI: (codec[0], codec[1]), orc.LO: (codec[2], codec[3])}
    seen = {orc.HI: 0, orc.LO: 0}
    for h in range(H):
        for tier, slot, rec in st.unit_tokens(0, h):
            p = rec["pos"]
            seen[tier] += 1
            for name, x, bits in (("k", k, widths[tier][0]), ("v", v, widths[tier][1])):
                xs = x[p, h].astype(np.float32)
                s16, z16 = (int(x) for x in rec[name + "meta"])
                step = float(np.uint16(s16).view(np.float16))
                codes = rec[name]
                assert codes.max() <= (1 << bits) - 1
                xh = np.array([orc.dequant(s16, z16, int(q)) for q in codes])
                rng_ = float(xs.max() - xs.min())
                bound = step / 2 * (1 + 1e-6) + ((1 << bits) - 1) * abs(step - rng_ / ((1 << bits) - 1)) + 1e-6
                assert np.all(np.abs(xh - xs) <= bound), (tier, name, np.abs(xh - xs).max(), bound)
    assert seen[orc.HI] > 0 and seen[orc.LO] > 0
