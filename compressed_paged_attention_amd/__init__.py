"""Python binding of libdiffkv.so (the MI355X DiffKV hot path).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch provides device memory and the current stream.  The C entry
points keep their names (``diffkv_classify``, ``diffkv_compact``,
``diffkv_decode_attn`` ...); ``DiffKVState`` only allocates the caller-owned
device buffers those calls work on.

The library must be built (``python -m compressed_paged_attention_amd.build``
or ``__graft_entry__.build()``); importing a missing library raises instead of
falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdiffkv.so")

DIFFKV_OK, DIFFKV_E_INVALID, DIFFKV_E_WORKSPACE, DIFFKV_E_HIP = 0, 1, 2, 3
ST_POOL_EXHAUSTED, ST_TABLE_OVERFLOW, ST_BAD_STATE, ST_STALE_CHAIN = 1, 2, 4, 8
PROMPT, STEP, RELEASE, ATTN, ATTN_SCORES, DECODE_STEP, DECODE_STEP_SCORES, IMPORTANCE, KEYDIFF = range(9)
IMP_CAUSAL, IMP_PROBE = 0, 1
PRUNE, LO, HI = 0, 1, 2


class DiffKVError(RuntimeError):
    pass


class diffkv_config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("gqa_group", ctypes.c_int32), ("hi_page_tokens", ctypes.c_int32),
                ("lo_page_tokens", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("window", ctypes.c_int32), ("lo_enabled", ctypes.c_int32),
                ("alpha_h", ctypes.c_float), ("alpha_l", ctypes.c_float),
                ("prompt_rule", ctypes.c_int32), ("alpha_h_head", ctypes.c_void_p),
                ("alpha_l_head", ctypes.c_void_p),
                ("hi_k_bits", ctypes.c_int32), ("hi_v_bits", ctypes.c_int32),
                ("lo_k_bits", ctypes.c_int32), ("lo_v_bits", ctypes.c_int32),
                ("num_levels", ctypes.c_int32), ("alpha_mid", ctypes.c_float * 2),
                ("mid_k_bits", ctypes.c_int32 * 2), ("mid_v_bits", ctypes.c_int32 * 2)]


RULE_ALPHA_N, RULE_ALPHA_I = 0, 1


class diffkv_pool(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("free_list", ctypes.c_void_p),
                ("ptr", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("num_pages", ctypes.c_int64), ("page_bytes", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libdiffkv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DiffKVError(f"{LIB_PATH} is missing: build it with "
                              "`python -m compressed_paged_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cfgp = ctypes.POINTER(diffkv_config)
        poolp = ctypes.POINTER(diffkv_pool)
        L.diffkv_page_bytes.argtypes = [cfgp]
        L.diffkv_page_bytes.restype = i32
        L.diffkv_table_len.argtypes = [cfgp]
        L.diffkv_table_len.restype = i32
        L.diffkv_state_words.argtypes = [cfgp]
        L.diffkv_state_words.restype = i32
        L.diffkv_attn_splits.argtypes = [cfgp, i32]
        L.diffkv_attn_splits.restype = i32
        L.diffkv_workspace_bytes.argtypes = [cfgp, i32, i32, i64]
        L.diffkv_workspace_bytes.restype = sz
        L.diffkv_pool_init.argtypes = [cfgp, poolp, vp]
        L.diffkv_state_init.argtypes = [cfgp, i32, vp, vp, vp]
        L.diffkv_classify.argtypes = [cfgp, i32, i64, vp, vp, vp, vp, vp]
        L.diffkv_compact.argtypes = [cfgp, poolp, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, sz, vp]
        L.diffkv_decode_attn.argtypes = [cfgp, poolp, i32, vp, vp, vp, vp, vp, i32, vp, sz, vp]
        L.diffkv_update_scores.argtypes = [cfgp, poolp, i32, vp, vp, vp, vp, sz, vp]
        L.diffkv_decode_step.argtypes = [cfgp, poolp, i32, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, sz, vp]
        L.diffkv_decode_attn_noalloc.argtypes = [cfgp, poolp, i32, vp, vp, vp, vp, vp, i32, vp]
        L.diffkv_importance.argtypes = [cfgp, i32, i32, i64, vp, i32, vp, vp, vp, vp, sz, vp]
        L.diffkv_keydiff_scores.argtypes = [cfgp, i32, i64, vp, vp, i32, vp, vp, sz, vp]
        L.diffkv_page_bounds.argtypes = [cfgp, poolp, i32, vp, vp, vp, vp]
        L.diffkv_page_scores.argtypes = [cfgp, poolp, i32, vp, vp, vp, vp, vp, vp, vp]
        for f in ("diffkv_pool_init", "diffkv_state_init", "diffkv_classify", "diffkv_compact",
                  "diffkv_decode_attn", "diffkv_update_scores", "diffkv_decode_step",
                  "diffkv_decode_attn_noalloc", "diffkv_importance", "diffkv_keydiff_scores",
                  "diffkv_page_bounds", "diffkv_page_scores"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


_head_alpha_cache: dict = {}


def _head_alphas(v, H: int):
    """Per-head thresholds as a device float32 tensor of H (cached by value,
    so a config reused across calls uploads them once)."""
    if isinstance(v, torch.Tensor):
        if not v.is_cuda or v.dtype != torch.float32 or not v.is_contiguous() or v.numel() != H:
            raise DiffKVError("per-head thresholds: contiguous float32 device tensor of H expected")
        return v
    key = (tuple(float(x) for x in v), torch.cuda.current_device())
    t = _head_alpha_cache.get(key)
    if t is None:
        if len(key[0]) != H:
            raise DiffKVError(f"per-head thresholds: {H} values expected")
        t = torch.tensor(key[0], dtype=torch.float32, device="cuda")
        _head_alpha_cache[key] = t
    return t


def make_config(c: dict) -> diffkv_config:
    """Config dict -> diffkv_config.  Optional keys: prompt_rule
    (RULE_ALPHA_N / RULE_ALPHA_I), alpha_h_head / alpha_l_head (H values
    each: a sequence, or a float32 device tensor) and hi_k_bits / hi_v_bits /
    lo_k_bits / lo_v_bits (tier codecs), num_levels (3 or 4 precision levels)
    with alpha_mid / mid_k_bits / mid_v_bits (one value per middle level)."""
    r = diffkv_config(int(c["head_dim"]), int(c["num_kv_heads"]), int(c["gqa_group"]),
                      int(c.get("hi_page_tokens", 16)), int(c.get("lo_page_tokens", 32)),
                      int(c["max_seq_len"]), int(c["window"]), int(c.get("lo_enabled", 1)),
                      float(c["alpha_h"]), float(c["alpha_l"]), int(c.get("prompt_rule", RULE_ALPHA_N)))
    keep = []
    for key in ("alpha_h_head", "alpha_l_head"):
        if c.get(key) is not None:
            t = _head_alphas(c[key], r.num_kv_heads)
            keep.append(t)
            setattr(r, key, t.data_ptr())
    r._keep = keep  # the device arrays live as long as the struct
    for key in ("hi_k_bits", "hi_v_bits", "lo_k_bits", "lo_v_bits"):  # tier codecs (absent: K8V4 / K4V2)
        setattr(r, key, int(c.get(key, 0)))
    r.num_levels = int(c.get("num_levels", 0))  # 3 or 4 precision levels (absent: two tiers)
    for key, conv in (("alpha_mid", float), ("mid_k_bits", int), ("mid_v_bits", int)):
        vals = list(c.get(key, ()))
        arr = getattr(r, key)
        for i in range(2):
            arr[i] = conv(vals[i]) if i < len(vals) else conv(0)
    return r


def _ptr(t) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda:
        raise DiffKVError("device tensor expected")
    if not t.is_contiguous():
        raise DiffKVError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, what: str):
    if rc != DIFFKV_OK:
        raise DiffKVError(f"{what} failed with code {rc}")


def diffkv_page_bytes(cfg: dict) -> int:
    return lib().diffkv_page_bytes(ctypes.byref(make_config(cfg)))


def diffkv_table_len(cfg: dict) -> int:
    return lib().diffkv_table_len(ctypes.byref(make_config(cfg)))


def diffkv_state_words(cfg: dict) -> int:
    return lib().diffkv_state_words(ctypes.byref(make_config(cfg)))


def diffkv_attn_splits(cfg: dict, batch: int) -> int:
    return lib().diffkv_attn_splits(ctypes.byref(make_config(cfg)), batch)


def diffkv_workspace_bytes(cfg: dict, op: int, batch: int, total_tokens: int = 0) -> int:
    return lib().diffkv_workspace_bytes(ctypes.byref(make_config(cfg)), op, batch, total_tokens)


class Pool:
    """Caller-owned device buffers of one page pool (torch allocations)."""

    def __init__(self, cfg: dict, num_pages: int, device="cuda"):
        self.cfg = dict(cfg)
        self.num_pages = int(num_pages)
        self.page_bytes = diffkv_page_bytes(cfg)
        if self.page_bytes <= 0:
            raise DiffKVError("invalid config")
        self.pages = torch.empty(self.num_pages * self.page_bytes, dtype=torch.uint8, device=device)
        self.free_list = torch.empty(self.num_pages, dtype=torch.int32, device=device)
        self.ptr = torch.empty(2, dtype=torch.int64, device=device)
        self.status = torch.empty(1, dtype=torch.int32, device=device)

    def struct(self) -> diffkv_pool:
        return diffkv_pool(self.pages.data_ptr(), self.free_list.data_ptr(), self.ptr.data_ptr(),
                           self.status.data_ptr(), self.num_pages, self.page_bytes)


def diffkv_pool_init(cfg: dict, pool: Pool, stream=None):
    _check(lib().diffkv_pool_init(ctypes.byref(make_config(cfg)), ctypes.byref(pool.struct()),
                                  _stream(stream)), "diffkv_pool_init")


def diffkv_state_init(cfg: dict, batch: int, page_table, tier_state, stream=None):
    _check(lib().diffkv_state_init(ctypes.byref(make_config(cfg)), batch, _ptr(page_table),
                                   _ptr(tier_state), _stream(stream)), "diffkv_state_init")


def diffkv_classify(cfg: dict, cu_seqlens, scores, tiers, tier_counts, total_tokens: int, stream=None):
    batch = cu_seqlens.numel() - 1
    _check(lib().diffkv_classify(ctypes.byref(make_config(cfg)), batch, int(total_tokens),
                                 _ptr(cu_seqlens), _ptr(scores), _ptr(tiers), _ptr(tier_counts),
                                 _stream(stream)), "diffkv_classify")


def diffkv_compact(cfg: dict, pool: Pool, mode: int, batch: int, page_table, tier_state, workspace,
                   total_tokens: int = 0, cu_seqlens=None, seq_len=None, k=None, v=None, scores=None,
                   tiers=None, release_mask=None, stream=None):
    _check(lib().diffkv_compact(ctypes.byref(make_config(cfg)), ctypes.byref(pool.struct()), mode, batch,
                                int(total_tokens), _ptr(cu_seqlens), _ptr(seq_len), _ptr(k), _ptr(v),
                                _ptr(scores), _ptr(tiers), _ptr(release_mask), _ptr(page_table),
                                _ptr(tier_state), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)), "diffkv_compact")


def diffkv_decode_attn(cfg: dict, pool: Pool, batch: int, q, page_table, tier_state, seq_len, out,
                       update_scores: int, workspace, stream=None):
    _check(lib().diffkv_decode_attn(ctypes.byref(make_config(cfg)), ctypes.byref(pool.struct()), batch,
                                    _ptr(q), _ptr(page_table), _ptr(tier_state), _ptr(seq_len), _ptr(out),
                                    int(update_scores), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)),
           "diffkv_decode_attn")


def diffkv_importance(cfg: dict, mode: int, cu_seqlens, q, k, scores, workspace, nq: int = 0, stream=None):
    """Prompt-phase importance (mean received attention, max over the group)
    into scores [H, total]; q: [total, H*G, d] (IMP_CAUSAL) or
    [batch, nq, H*G, d] (IMP_PROBE), k: [total, H, d] fp16 bits."""
    batch = cu_seqlens.numel() - 1
    total = int(k.shape[0])
    _check(lib().diffkv_importance(ctypes.byref(make_config(cfg)), int(mode), batch, total, _ptr(cu_seqlens),
                                   int(nq), _ptr(q), _ptr(k), _ptr(scores), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "diffkv_importance")


def importance(cfg: dict, cu_seqlens, q, k, nq: int = 0):
    """Allocates the outputs and workspace (torch) and calls diffkv_importance:
    causal from the prompt's own queries, or from probes when nq > 0."""
    total = int(k.shape[0])
    H = int(cfg["num_kv_heads"])
    batch = cu_seqlens.numel() - 1
    mode = IMP_PROBE if nq > 0 else IMP_CAUSAL
    n = batch * nq if nq > 0 else total
    ws = torch.empty(max(diffkv_workspace_bytes(cfg, IMPORTANCE, batch, n), 256), dtype=torch.uint8, device=k.device)
    scores = torch.empty(H, total, dtype=torch.float32, device=k.device)
    diffkv_importance(cfg, mode, cu_seqlens, q, k, scores, ws, nq=nq)
    return scores


def keydiff_scores(cfg: dict, cu_seqlens, k, anchor_raw: bool = False):
    """Query-free importance from the keys (diffkv_keydiff_scores): allocates
    the outputs and workspace (torch); fp32 [H, total]."""
    total = int(k.shape[0])
    batch = cu_seqlens.numel() - 1
    ws = torch.empty(diffkv_workspace_bytes(cfg, KEYDIFF, batch, total), dtype=torch.uint8, device=k.device)
    scores = torch.empty(int(cfg["num_kv_heads"]), total, dtype=torch.float32, device=k.device)
    _check(lib().diffkv_keydiff_scores(ctypes.byref(make_config(cfg)), batch, total, _ptr(cu_seqlens), _ptr(k),
                                       1 if anchor_raw else 0, _ptr(scores), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(None)), "diffkv_keydiff_scores")
    return scores


NOALLOC_SCRATCH_BYTES = 64 << 20


def diffkv_decode_attn_noalloc(cfg: dict, pool: Pool, batch: int, q, page_table, tier_state, seq_len, out,
                               update_scores: int, stream=None) -> int:
    """Returns the library's code (DIFFKV_OK or an error) instead of raising,
    so callers can see the size limit's DIFFKV_E_WORKSPACE."""
    return lib().diffkv_decode_attn_noalloc(ctypes.byref(make_config(cfg)), ctypes.byref(pool.struct()), batch,
                                            _ptr(q), _ptr(page_table), _ptr(tier_state), _ptr(seq_len), _ptr(out),
                                            int(update_scores), _stream(stream))


def diffkv_update_scores(cfg: dict, pool: Pool, batch: int, page_table, tier_state, seq_len, workspace,
                         stream=None):
    _check(lib().diffkv_update_scores(ctypes.byref(make_config(cfg)), ctypes.byref(pool.struct()), batch,
                                      _ptr(page_table), _ptr(tier_state), _ptr(seq_len), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)),
           "diffkv_update_scores")


def diffkv_decode_step(cfg: dict, pool: Pool, batch: int, seq_len, k_new, v_new, q, page_table, tier_state,
                       out, update_scores: int, workspace, chain: int = 0, stream=None):
    _check(lib().diffkv_decode_step(ctypes.byref(make_config(cfg)), ctypes.byref(pool.struct()), batch,
                                    _ptr(seq_len), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(page_table),
                                    _ptr(tier_state), _ptr(out), int(update_scores), int(chain), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)),
           "diffkv_decode_step")


class DiffKVState:
    """All device buffers of one cache (pool, tables, workspaces) for `batch` slots."""

    def __init__(self, cfg: dict, batch: int, num_pages: int, max_total_tokens: int = 0, device="cuda"):
        self.cfg = dict(cfg)
        self.batch = batch
        self.H = int(cfg["num_kv_heads"])
        self.G = int(cfg["gqa_group"])
        self.d = int(cfg["head_dim"])
        self.L = diffkv_table_len(cfg)
        self.pool = Pool(cfg, num_pages, device)
        self.page_table = torch.empty(batch, self.H, self.L, dtype=torch.int32, device=device)
        self.K = diffkv_state_words(cfg) // 2  # precision levels
        self.tier_state = torch.empty(batch, self.H, 2 * self.K, dtype=torch.int32, device=device)
        cws = max(diffkv_workspace_bytes(cfg, PROMPT, batch, max_total_tokens),
                  diffkv_workspace_bytes(cfg, STEP, batch), diffkv_workspace_bytes(cfg, RELEASE, batch))
        self.ws_compact = torch.empty(cws, dtype=torch.uint8, device=device)
        self.ws_attn = torch.zeros(diffkv_workspace_bytes(cfg, ATTN_SCORES, batch), dtype=torch.uint8,
                                   device=device)
        self.ws_decode = torch.zeros(diffkv_workspace_bytes(cfg, DECODE_STEP_SCORES, batch), dtype=torch.uint8,
                                     device=device)
        diffkv_pool_init(cfg, self.pool)
        diffkv_state_init(cfg, batch, self.page_table, self.tier_state)
        # decode_step(update_scores=1) calls made in a row (their attention
        # leaves the next step's plans in ws_decode); any other call that
        # writes the cache ends the chain
        self.chain = 0

    def classify(self, cu_seqlens, scores):
        total = int(scores.shape[1])
        tiers = torch.empty(self.H, total, dtype=torch.uint8, device=scores.device)
        counts = torch.empty(cu_seqlens.numel() - 1, self.H, self.K, dtype=torch.int32, device=scores.device)
        diffkv_classify(self.cfg, cu_seqlens, scores, tiers, counts, total)
        return tiers, counts

    def compact_prompt(self, cu_seqlens, k, v, scores, tiers):
        total = int(scores.shape[1])
        need = diffkv_workspace_bytes(self.cfg, PROMPT, self.batch, total)
        if self.ws_compact.numel() < need:
            self.ws_compact = torch.empty(need, dtype=torch.uint8, device=self.ws_compact.device)
        self.chain = 0
        diffkv_compact(self.cfg, self.pool, PROMPT, self.batch, self.page_table, self.tier_state,
                       self.ws_compact, total_tokens=total, cu_seqlens=cu_seqlens, k=k, v=v,
                       scores=scores, tiers=tiers)

    def compact_step(self, seq_len, k_new, v_new):
        self.chain = 0
        diffkv_compact(self.cfg, self.pool, STEP, self.batch, self.page_table, self.tier_state,
                       self.ws_compact, seq_len=seq_len, k=k_new, v=v_new)

    def release(self, mask):
        self.chain = 0
        diffkv_compact(self.cfg, self.pool, RELEASE, self.batch, self.page_table, self.tier_state,
                       self.ws_compact, release_mask=mask)

    def decode_attn(self, q, seq_len, update_scores: int = 0, out=None):
        if out is None:
            out = torch.empty(self.batch, self.H * self.G, self.d, dtype=torch.float32, device=q.device)
        if update_scores:
            self.chain = 0
        diffkv_decode_attn(self.cfg, self.pool, self.batch, q, self.page_table, self.tier_state, seq_len,
                           out, int(update_scores), self.ws_attn)
        return out

    def decode_step(self, q, seq_len, k_new, v_new, update_scores: int = 1, out=None, chain=None):
        """compact_step(seq_len, k_new, v_new) then decode_attn(q, seq_len), as one call.

        chain: None follows this object's own count of decode_step calls
        made in a row (0 forces the plan kernel)."""
        if out is None:
            out = torch.empty(self.batch, self.H * self.G, self.d, dtype=torch.float32, device=q.device)
        c = self.chain if chain is None else int(chain)
        self.chain = 0
        diffkv_decode_step(self.cfg, self.pool, self.batch, seq_len, k_new, v_new, q, self.page_table,
                           self.tier_state, out, int(update_scores), self.ws_decode,
                           chain=c if update_scores == 1 else 0)
        if update_scores == 1:
            self.chain = c + 1
        return out

    def page_bounds(self, bounds=None):
        """Per-page key bounds [num_pages, 2, d] fp32 (min row, max row) of
        every live page (diffkv_page_bounds); other rows as they were."""
        if bounds is None:
            bounds = torch.full((self.pool.num_pages, 2, self.d), float("nan"), dtype=torch.float32,
                                device=self.page_table.device)
        _check(lib().diffkv_page_bounds(ctypes.byref(make_config(self.cfg)), ctypes.byref(self.pool.struct()),
                                        self.batch, _ptr(self.page_table), _ptr(self.tier_state), _ptr(bounds),
                                        _stream(None)), "diffkv_page_bounds")
        return bounds

    def page_scores(self, q, seq_len, bounds):
        """Page scores [batch, H, table_len] in table order (diffkv_page_scores)."""
        out = torch.empty(self.batch, self.H, self.L, dtype=torch.float32, device=q.device)
        _check(lib().diffkv_page_scores(ctypes.byref(make_config(self.cfg)), ctypes.byref(self.pool.struct()),
                                        self.batch, _ptr(q), _ptr(self.page_table), _ptr(self.tier_state),
                                        _ptr(seq_len), _ptr(bounds), _ptr(out), _stream(None)),
               "diffkv_page_scores")
        return out

    def update_scores(self, seq_len):
        self.chain = 0
        diffkv_update_scores(self.cfg, self.pool, self.batch, self.page_table, self.tier_state, seq_len,
                             self.ws_attn)
