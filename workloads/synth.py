"""Seeded synthetic inputs shaped like the DiffKV workloads.

The notes evaluate on Llama3 / Qwen2.5 / QwQ models over MATH, AIME24,
GSM8K, HumanEval+, LongBench and GPQA; none of those weights or datasets is
used.  These generators stand in for them:

* K and V: fp16 (round to nearest even of fp32 draws) N(0, 1) times a
  per-(KV head, channel) scale where a few outlier channels are x8;
* importance (mean received attention) per token: a Zipf(s) mass over ranks
  1..N, ranks randomly permuted per (request, KV head); or, for the tiny
  case, raw probe queries whose attention the oracle turns into scores;
* decode queries N(0, 1) fp16; new K/V rows drawn like the prompt's.

Generation runs in torch on the requested device with a seeded generator
(seed = 20261202 + config id), so large cases are drawn on the GPU; values
drawn on different devices differ, the recipe does not.  Arrays hold fp16 as
raw uint16 bits (torch.int16 views) so both bindings receive plain bits.
"""
from __future__ import annotations

import math

import torch

SEED_BASE = 20261202

# Workload table.  Sizes, GQA shapes and thresholds follow the configs the
# build is measured on; alpha_h = 1.0, alpha_l = 0.2 throughout.
CONFIGS = {
    "tiny": dict(cid=1, head_dim=64, num_kv_heads=4, gqa_group=2, batch=1,
                 seq=(256, 256), score="probe", nprobe=16, outliers=2,
                 alpha_h=1.0, alpha_l=0.2, window=64, lo_enabled=1,
                 num_pages=64, max_seq_len=512),
    "llama3_8b": dict(cid=2, head_dim=128, num_kv_heads=8, gqa_group=4, batch=32,
                      seq=(4096, 4096), score="zipf", zipf=(1.1, 1.1), outliers=4,
                      alpha_h=1.0, alpha_l=0.2, window=64, lo_enabled=1,
                      pool_factor=1.25, max_seq_len=4096 + 256),
    "long": dict(cid=3, head_dim=128, num_kv_heads=8, gqa_group=4, batch=8,
                 seq=(32768, 32768), score="zipf", zipf=(0.6, 1.6), outliers=4,
                 alpha_h=1.0, alpha_l=0.2, window=64, lo_enabled=1,
                 pool_factor=1.25, max_seq_len=32768 + 256),
    "churn": dict(cid=4, head_dim=128, num_kv_heads=8, gqa_group=5, batch=128,
                  seq=(1000, 16000), score="zipf", zipf=(1.1, 1.1), outliers=4,
                  alpha_h=1.0, alpha_l=0.2, window=64, lo_enabled=1,
                  steps=256, budget=(1, 512), pool_factor=1.3,
                  max_seq_len=16000 + 512 + 16),
    "stress_gqa7": dict(cid=5, head_dim=128, num_kv_heads=4, gqa_group=7, batch=64,
                        seq=(2000, 64000), score="zipf", zipf=(1.1, 1.1), outliers=4,
                        alpha_h=1.0, alpha_l=0.2, window=64, lo_enabled=0,
                        pool_bytes=200 * 10**9, max_seq_len=64000 + 256),
    "stress_gqa8": dict(cid=6, head_dim=128, num_kv_heads=8, gqa_group=8, batch=64,
                        seq=(2000, 64000), score="zipf", zipf=(1.1, 1.1), outliers=4,
                        alpha_h=1.0, alpha_l=0.2, window=64, lo_enabled=1,
                        pool_bytes=200 * 10**9, max_seq_len=64000 + 256),
}


def config(name: str, **over) -> dict:
    c = dict(CONFIGS[name])
    c.update(over)
    c.setdefault("hi_page_tokens", 16)
    c.setdefault("lo_page_tokens", 32)
    c["name"] = name
    return c


def _gen(cfg: dict, salt: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(SEED_BASE + 1000 * int(cfg["cid"]) + salt)
    return g


def seq_lens(cfg: dict, device="cpu", salt: int = 0) -> torch.Tensor:
    lo, hi = cfg["seq"]
    B = cfg["batch"]
    if lo == hi:
        return torch.full((B,), lo, dtype=torch.int64)
    g = _gen(cfg, 1 + salt, "cpu")
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)


def channel_scale(cfg: dict, device="cpu") -> torch.Tensor:
    """[H, d] fp32: 1 everywhere except `outliers` random channels per head at 8."""
    H, d = cfg["num_kv_heads"], cfg["head_dim"]
    g = _gen(cfg, 2, "cpu")
    sc = torch.ones(H, d)
    for h in range(H):
        idx = torch.randperm(d, generator=g)[: cfg["outliers"]]
        sc[h, idx] = 8.0
    return sc.to(device)


def _f16_bits(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.float16).view(torch.int16)


def zipf_scores(cfg: dict, lens: torch.Tensor, device="cpu", salt: int = 0) -> torch.Tensor:
    """[H, sum N] fp32 Zipf(s) attention mass per token, ranks permuted per unit."""
    H = cfg["num_kv_heads"]
    total = int(lens.sum())
    out = torch.empty(H, total, dtype=torch.float32, device=device)
    g = _gen(cfg, 3 + salt, device)
    gs = _gen(cfg, 4 + salt, "cpu")
    s_lo, s_hi = cfg["zipf"]
    off = 0
    for r, n in enumerate(lens.tolist()):
        for h in range(H):
            s = s_lo if s_lo == s_hi else float(torch.empty(1).uniform_(s_lo, s_hi, generator=gs))
            ranks = torch.arange(1, n + 1, dtype=torch.float64, device=device)
            mass = ranks.pow(-s)
            mass = mass / mass.sum()
            perm = torch.randperm(n, generator=g, device=device)
            out[h, off:off + n] = mass[perm].to(torch.float32)
        off += n
    return out


def probe_queries(cfg: dict, device="cpu") -> torch.Tensor:
    """[B, nprobe, H*G, d] fp16 bits: random probe queries for the tiny case."""
    g = _gen(cfg, 5, device)
    B, H, G, d = cfg["batch"], cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    q = torch.randn(B, cfg["nprobe"], H * G, d, generator=g, device=device)
    return _f16_bits(q)


def make_prompt(cfg: dict, device="cpu", salt: int = 0, lens: torch.Tensor | None = None) -> dict:
    """Prompt K/V ([sum N, H, d] fp16 bits), cu_seqlens and Zipf scores if any."""
    if lens is None:
        lens = seq_lens(cfg, salt=salt)
    H, d = cfg["num_kv_heads"], cfg["head_dim"]
    total = int(lens.sum())
    cu = torch.zeros(lens.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    g = _gen(cfg, 10 + salt, device)
    sc = channel_scale(cfg, device)
    k = torch.randn(total, H, d, generator=g, device=device) * sc
    k = _f16_bits(k)
    v = torch.randn(total, H, d, generator=g, device=device) * sc
    v = _f16_bits(v)
    out = dict(lens=lens, cu_seqlens=cu, k=k, v=v)
    if cfg["score"] == "zipf":
        out["scores"] = zipf_scores(cfg, lens, device, salt)
    return out


def make_decode(cfg: dict, step: int, device="cpu", batch: int | None = None, q_scale: float = 1.0) -> dict:
    """One decode step's inputs: q [B, H*G, d], k_new / v_new [B, H, d] (fp16 bits).
    q_scale multiplies the query draws (a sharper softmax: a few tokens take
    most of the weight, the rest lose importance step by step)."""
    B = cfg["batch"] if batch is None else batch
    H, G, d = cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    g = _gen(cfg, 100 + step, device)
    sc = channel_scale(cfg, device)
    q = _f16_bits(torch.randn(B, H * G, d, generator=g, device=device) * q_scale)
    kn = _f16_bits(torch.randn(B, H, d, generator=g, device=device) * sc)
    vn = _f16_bits(torch.randn(B, H, d, generator=g, device=device) * sc)
    return dict(q=q, k_new=kn, v_new=vn)


def pool_pages(cfg: dict, lens: torch.Tensor, page_bytes: int) -> int:
    """Pool size: a factor over the conservative prompt need, or a byte budget."""
    if "num_pages" in cfg:
        return int(cfg["num_pages"])
    if "pool_bytes" in cfg:
        return int(cfg["pool_bytes"] // page_bytes)
    need = sum(math.ceil(n / cfg["hi_page_tokens"]) for n in lens.tolist()) * cfg["num_kv_heads"]
    return int(math.ceil(need * cfg["pool_factor"]))
